"""The C-ABI calls captured in a HIP graph give the eager result on every replay.

The library enqueues only kernels on the caller's stream (no memsets, no
allocations), so a captured fwd+bwd step must replay to the same bits as the
eager call; replays are interleaved with eager work and synchronisation.
"""
import numpy as np
import pytest
import torch

from evoformer_biased_attention_amd import inputs as I
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_row", "msa_row"])
def test_graph_replay_matches_eager(name):
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd

    cfg = I.CONFIGS[name]
    print(f"case graph replay {name} shape={cfg.shape}", flush=True)
    bits = I.make_inputs(cfg)
    q, k, v, m, p, do = (to_device(bits[n], cfg.dtype) for n in ("q", "k", "v", "mask_bias", "pair_bias", "dout"))
    out_e, lse_e = attn_fwd(q, k, v, m, p)
    g_e = attn_bwd(q, k, v, m, p, out_e, lse_e, do)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out_e, lse_e, g_e["dq"], g_e["dk"], g_e["dv"], g_e["dmask"], g_e["dpair"])]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn_fwd(q, k, v, m, p)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g, lse_g = attn_fwd(q, k, v, m, p)
        g_g = attn_bwd(q, k, v, m, p, out_g, lse_g, do)
    got = (out_g, lse_g, g_g["dq"], g_g["dk"], g_g["dv"], g_g["dmask"], g_g["dpair"])
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(got, ref):
            assert torch.equal(a_, b_), f"replay {rep} differs"
        # eager work between replays
        attn_fwd(q, k, v, m, p)
        torch.cuda.synchronize()
