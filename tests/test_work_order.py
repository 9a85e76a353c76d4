"""The forward's balanced work order, checked on the host.

balanced_unit_rank (evo_kernels.h) maps each logical workgroup slot to the
rank of the work unit it runs when batch entries of mixed live length are
reordered.  tests/host/work_order_check.hip includes that header, is built
with hipcc for the host here, and checks the mapping over 2048 grid shapes:
a bijection onto the ranks, one rank per unit, and complementary ranks for the
two workgroups that share a CU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from evoformer_biased_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "work_order_check.hip")


@pytest.mark.timeout(300)
def test_balanced_unit_rank_is_a_complementary_bijection():
    if shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not installed")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "work_order_check")
        r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", B.INCLUDE, "-I", B.CSRC,
                            SRC, "-o", exe], capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("ok: 2048"), r.stdout
