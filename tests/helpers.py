"""Shared test helpers: seeded inputs onto the GPU, oracle comparison.

Nothing here computes attention: the GPU side calls the C ABI through the
package binding, the expected side calls oracle/ only.
"""
from __future__ import annotations

import numpy as np
import torch

from evoformer_biased_attention_amd import inputs as I

TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}
# tolerances (max abs error): outputs / gradients per dtype; lse is fp32
TOL = {"fp16": {"out": 5e-3, "grad": 2e-2}, "bf16": {"out": 2e-2, "grad": 5e-2}}
LSE_TOL = 1e-3


def to_device(bits, dtype, device="cuda"):
    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(TORCH_DT[dtype])


def to_f64(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def rne_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> dtype bits, round to nearest even (numpy cast / bit arithmetic)."""
    return I.to_bits(np.asarray(x32, np.float32), dtype)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))
