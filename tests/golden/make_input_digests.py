"""Write input_digests.json: sha256 of the seeded synthetic inputs (no oracle, no GPU)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from evoformer_biased_attention_amd import inputs as I  # noqa: E402

out = {name: I.digest(I.make_inputs(I.CONFIGS[name])) for name in ("tiny_row",)}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json"), "w") as f:
    json.dump(out, f, indent=1)
