"""The C-ABI library: exported symbols and host-side argument checks (CPU), error paths (GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

from evoformer_biased_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "evo_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(evo_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(0, 13):
        assert _lib.evo_status_string(s)
    assert _lib.evo_status_string(99) == "unknown status"


@pytest.mark.parametrize("shape,dtype,code", [
    ((1, 2, 32, 2, 7), 0, 4),     # head dim
    ((1, 2, 32, 2, 128), 0, 4),
    ((0, 2, 32, 2, 32), 0, 2),    # empty dim
    ((1, 2, -3, 2, 32), 1, 2),
    ((1, 2, 32, 2, 32), 2, 3),    # dtype
    ((1, 2, 65537, 2, 32), 0, 2),  # L beyond 65536
    ((1, 1, 65536, 512, 64), 0, 2),  # one slice past 2 GiB (32-bit tile offsets)
])
def test_argument_errors_are_reported_before_any_device_call(shape, dtype, code):
    # these fail in shape/dtype parsing, before the library touches the device
    assert _lib.evo_attn_fwd(None, None, None, None, None, None, None, shape, dtype, None) == code
    assert _lib.evo_attn_bwd(*([None] * 14), 0, shape, dtype, None) == code
    assert _lib.evo_attn_bwd_workspace_bytes(shape, dtype, 1, 1) == 0


def test_workspace_size_and_layout_host_logic():
    shape = (1, 16, 32, 2, 8)
    full = _lib.evo_attn_bwd_workspace_bytes(shape, 0, 1, 1)
    none = _lib.evo_attn_bwd_workspace_bytes(shape, 0, 0, 0)
    assert full > none >= 1 * 16 * 2 * 32 * 4
    od, om, op = _lib.evo_attn_bwd_workspace_offsets(shape, 0, 1, 1)
    assert od == 0 and om is not None and op is not None
    assert op + 1 * 2 * 32 * 32 * 4 <= full
    od, om, op = _lib.evo_attn_bwd_workspace_offsets(shape, 0, 0, 0)
    assert om is None and op is None


@pytest.mark.parametrize("strides,code", [
    ((8, 8, 7), 11),          # not a multiple of 8 elements
    ((0, 64, 16), 11),        # not positive
    ((1024, 64, 8), 11),      # L rows overlap: sL < H * D
    ((1024, 32, 16), 11),     # N rows overlap the span of the L rows
    ((2048, 16, 32), 1),      # transposed over N and L: valid (then the NULL pointers)
    ((2048, 1024, 32), 1),    # padded rows: valid
])
def test_layout_errors_are_reported_before_any_device_call(strides, code):
    shape = (2, 2, 32, 2, 8)  # H * D = 16
    assert _lib.evo_attn_fwd_strided(None, None, None, None, None, None, None, shape, strides, 0, None) == code
    assert _lib.evo_attn_bwd_strided(*([None] * 14), 0, shape, strides, 0, None) == code


def test_layout_slice_limit():
    # (L - 1) * sL + H * D elements of one slice must stay under 2 GiB
    shape = (1, 1, 65536, 1, 8)
    ok, bad = (1 << 40, 1 << 40, 16384), (1 << 40, 1 << 40, 16392)
    assert _lib.evo_attn_fwd_strided(None, None, None, None, None, None, None, shape, ok, 0, None) == 1
    assert _lib.evo_attn_fwd_strided(None, None, None, None, None, None, None, shape, bad, 0, None) == 11


_NO_DEVICE_PROBE = r"""
import sys
sys.path.insert(0, sys.argv[1])
from evoformer_biased_attention_amd import _lib
shape = (1, 2, 32, 2, 32)
p = [16 * (i + 1) for i in range(14)]  # non-NULL, aligned; never dereferenced
fwd = _lib.evo_attn_fwd(p[0], p[1], p[2], None, None, p[3], p[4], shape, _lib.EVO_F16, None)
nws = _lib.evo_attn_bwd_workspace_bytes(shape, _lib.EVO_F16, 0, 0)
bwd = _lib.evo_attn_bwd(p[0], p[1], p[2], None, None, p[3], p[4], p[5], p[6], p[7], p[8], None, None,
                        p[9], nws, shape, _lib.EVO_F16, None)
print(fwd, bwd)
"""


def test_no_usable_device_is_reported_as_evo_err_device():
    """With no HIP device visible to the process, valid arguments reach the
    library's device check (guide §3.7: inputs must live on the GPU the kernel
    was built for), which answers EVO_ERR_DEVICE and enqueues nothing."""
    import subprocess
    import sys

    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", _NO_DEVICE_PROBE, ROOT], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    fwd, bwd = (int(x) for x in r.stdout.split()[-2:])
    assert fwd == _lib.EVO_ERR_DEVICE and bwd == _lib.EVO_ERR_DEVICE, r.stdout


def test_noalloc_backward_refuses_problems_past_its_static_scratch():
    """evo_attn_bwd_noalloc works inside a static device array of
    EVO_NOALLOC_SCRATCH_BYTES; a problem whose least workspace is larger is
    refused with EVO_ERR_SCRATCH_LIMIT before any device call."""
    big = (1, 2048, 1024, 4, 32)  # delta and the dmask partials alone pass 64 MiB
    assert _lib.evo_attn_bwd_workspace_bytes_within(big, _lib.EVO_BF16, 1, 1, 0) > _lib.EVO_NOALLOC_SCRATCH_BYTES
    p = [16 * (i + 1) for i in range(13)]
    assert _lib.evo_attn_bwd_noalloc(*p, big, None, _lib.EVO_BF16, None) == _lib.EVO_ERR_SCRATCH_LIMIT
    # argument errors come first, as in evo_attn_bwd
    assert _lib.evo_attn_bwd_noalloc(*([None] * 13), (1, 2, 32, 2, 7), None, 0, None) == _lib.EVO_ERR_HEAD_DIM
    assert "EVO_NOALLOC_SCRATCH_BYTES" in _lib.evo_status_string(_lib.EVO_ERR_SCRATCH_LIMIT)


MiB = 1 << 20


@pytest.mark.parametrize("shape,has_pair", [((1, 768, 768, 4, 32), 1), ((1, 384, 512, 8, 32), 0),
                                            ((2, 48, 640, 2, 64), 1), ((1, 256, 256, 4, 32), 1)])
def test_backward_plan_fits_the_workspace(shape, has_pair):
    """The backward fits its plan to the workspace: more room for the fp32
    partials never gives a smaller workspace, the partials stay within the
    budget whenever some plan fits it, the default is the plan for 384 MiB of
    partials, and rows of one key tile, or longer rows without a pair bias
    (dQ kept in registers over the key tiles, no partials), do not depend on
    the budget at all."""
    dt = _lib.EVO_BF16
    within = lambda b: _lib.evo_attn_bwd_workspace_bytes_within(shape, dt, 1, has_pair, b)
    least = within(0)
    fixed = _lib.evo_attn_bwd_workspace_offsets(shape, dt, 1, has_pair)
    assert least > 0
    sizes = [within(b * MiB) for b in (0, 32, 64, 128, 160, 256, 384, 640, 4096)]
    assert sizes == sorted(sizes)
    assert _lib.evo_attn_bwd_workspace_bytes(shape, dt, 1, has_pair) == within(384 * MiB)
    B, N, L, H, D = shape
    jtiles = -(-L // (128 if D == 64 else 256))
    if jtiles == 1 or not has_pair:
        assert len(set(sizes)) == 1
        return
    # the regions that do not depend on the plan: delta, dmask partials and
    # accumulators, the dpair accumulator
    fixed_bytes = sum(-(-n // 256) * 256 for n in (B * N * H * L * 4, B * N * H * L * 4, B * N * L * 4,
                                                     (B * H * L * L * 4) if has_pair else 0))
    slot = B * H * L * L * 4 if has_pair else 0
    for b in (64, 128, 160, 256, 384, 640):
        got = within(b * MiB)
        # a plan that fits exists once one slice with one dpair slot does
        if jtiles * B * L * H * D * 4 + slot + 512 <= b * MiB:
            assert got - fixed_bytes <= b * MiB, (b, got)
    # offsets of the fp32 accumulators do not depend on the plan
    assert fixed[0] == 0


def test_triangle_workspace_bounds():
    """(1,768,768,4,32): the default plan keeps the long-row partials within
    384 MiB (the whole workspace under 450 MB), and 160 MiB of partials brings
    the workspace under 200 MB."""
    shape = (1, 768, 768, 4, 32)
    assert _lib.evo_attn_bwd_workspace_bytes(shape, _lib.EVO_BF16, 1, 1) < 450e6
    assert _lib.evo_attn_bwd_workspace_bytes_within(shape, _lib.EVO_BF16, 1, 1, 160 * MiB) < 200e6
