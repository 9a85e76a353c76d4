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
    for s in range(0, 11):
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
