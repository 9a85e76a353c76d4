"""ctypes binding of libevoattn.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libevoattn.so")

EVO_F16 = 0
EVO_BF16 = 1

# status codes (include/evo_attn.h)
EVO_OK = 0
EVO_ERR_NULL_POINTER = 1
EVO_ERR_BAD_SHAPE = 2
EVO_ERR_BAD_DTYPE = 3
EVO_ERR_HEAD_DIM = 4
EVO_ERR_ALIGNMENT = 5
EVO_ERR_NOT_DEVICE_MEMORY = 6
EVO_ERR_WORKSPACE = 7
EVO_ERR_DEVICE = 8
EVO_ERR_LAUNCH = 9
EVO_ERR_ALIAS = 10
EVO_ERR_BAD_STRIDES = 11
EVO_ERR_SCRATCH_LIMIT = 12
EVO_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = (
    "evo_attn_fwd",
    "evo_attn_bwd",
    "evo_attn_fwd_strided",
    "evo_attn_bwd_strided",
    "evo_attn_bwd_noalloc",
    "evo_attn_bwd_workspace_bytes",
    "evo_attn_bwd_workspace_bytes_within",
    "evo_attn_bwd_workspace_offsets",
    "evo_status_string",
    "evo_attn_profile_enable",
    "evo_attn_profile_read",
    "evo_attn_profile_kernel_name",
)
PROFILE_KINDS = 5

_lib: Optional[ctypes.CDLL] = None


class EvoError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"evo_attn status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m evoformer_biased_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I, Z = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_size_t
    lib.evo_attn_fwd.argtypes = [P, P, P, P, P, P, P, S, I, P]
    lib.evo_attn_fwd.restype = I
    lib.evo_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, S, I, P]
    lib.evo_attn_bwd.restype = I
    lib.evo_attn_fwd_strided.argtypes = [P, P, P, P, P, P, P, S, S, I, P]
    lib.evo_attn_fwd_strided.restype = I
    lib.evo_attn_bwd_strided.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, S, S, I, P]
    lib.evo_attn_bwd_strided.restype = I
    lib.evo_attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, S, S, I, P]
    lib.evo_attn_bwd_noalloc.restype = I
    lib.evo_attn_bwd_workspace_bytes.argtypes = [S, I, I, I]
    lib.evo_attn_bwd_workspace_bytes.restype = Z
    lib.evo_attn_bwd_workspace_bytes_within.argtypes = [S, I, I, I, Z]
    lib.evo_attn_bwd_workspace_bytes_within.restype = Z
    lib.evo_attn_bwd_workspace_offsets.argtypes = [S, I, I, I, ctypes.POINTER(Z), ctypes.POINTER(Z), ctypes.POINTER(Z)]
    lib.evo_attn_bwd_workspace_offsets.restype = I
    lib.evo_status_string.argtypes = [I]
    lib.evo_status_string.restype = ctypes.c_char_p
    lib.evo_attn_profile_enable.argtypes = [I]
    lib.evo_attn_profile_enable.restype = I
    lib.evo_attn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.evo_attn_profile_read.restype = I
    lib.evo_attn_profile_kernel_name.argtypes = [I]
    lib.evo_attn_profile_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def shape_arg(shape):
    return (ctypes.c_int64 * 5)(*[int(x) for x in shape])


def check(status: int) -> None:
    if status != 0:
        raise EvoError(status, load().evo_status_string(status).decode())


def evo_attn_fwd(q, k, v, mask_bias, pair_bias, out, lse, shape, dtype, stream) -> int:
    return load().evo_attn_fwd(q, k, v, mask_bias, pair_bias, out, lse, shape_arg(shape), dtype, stream)


def evo_attn_bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias,
                 workspace, workspace_bytes, shape, dtype, stream) -> int:
    return load().evo_attn_bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias,
                               dpair_bias, workspace, workspace_bytes, shape_arg(shape), dtype, stream)


def strides_arg(strides):
    return None if strides is None else (ctypes.c_int64 * 3)(*[int(x) for x in strides])


def evo_attn_fwd_strided(q, k, v, mask_bias, pair_bias, out, lse, shape, strides, dtype, stream) -> int:
    return load().evo_attn_fwd_strided(q, k, v, mask_bias, pair_bias, out, lse, shape_arg(shape),
                                       strides_arg(strides), dtype, stream)


def evo_attn_bwd_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias,
                         workspace, workspace_bytes, shape, strides, dtype, stream) -> int:
    return load().evo_attn_bwd_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias,
                                       dpair_bias, workspace, workspace_bytes, shape_arg(shape),
                                       strides_arg(strides), dtype, stream)


def evo_attn_bwd_noalloc(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias,
                         shape, strides, dtype, stream) -> int:
    return load().evo_attn_bwd_noalloc(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias,
                                       dpair_bias, shape_arg(shape), strides_arg(strides), dtype, stream)


def evo_attn_bwd_workspace_bytes(shape, dtype, has_mask, has_pair) -> int:
    return int(load().evo_attn_bwd_workspace_bytes(shape_arg(shape), dtype, int(has_mask), int(has_pair)))


def evo_attn_bwd_workspace_bytes_within(shape, dtype, has_mask, has_pair, partial_budget) -> int:
    return int(load().evo_attn_bwd_workspace_bytes_within(shape_arg(shape), dtype, int(has_mask), int(has_pair),
                                                          int(partial_budget)))


def evo_attn_bwd_workspace_offsets(shape, dtype, has_mask, has_pair):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    check(load().evo_attn_bwd_workspace_offsets(shape_arg(shape), dtype, int(has_mask), int(has_pair),
                                                ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    none = (1 << 64) - 1
    conv = lambda x: None if x.value == none else int(x.value)
    return conv(a), conv(b), conv(c)


def evo_status_string(status: int) -> str:
    return load().evo_status_string(status).decode()


def evo_attn_profile_enable(on: bool) -> bool:
    return bool(load().evo_attn_profile_enable(int(on)))


def evo_attn_profile_read():
    """{kernel name: (total_ms, launches)} since the previous read."""
    ms = (ctypes.c_double * PROFILE_KINDS)()
    n = (ctypes.c_int64 * PROFILE_KINDS)()
    check(load().evo_attn_profile_read(ms, n))
    return {load().evo_attn_profile_kernel_name(k).decode(): (float(ms[k]), int(n[k])) for k in range(PROFILE_KINDS)}
