"""Seeded synthetic inputs for Evoformer biased attention.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It draws random numbers and rounds them to the storage
dtype; it holds none of the attention arithmetic.

Shapes follow the DeepSpeed4Science guide (page "DeepSpeed4Science 技术指南",
§3.6, the usage examples of MSA row, MSA column and triangle attention):

* q, k, v, dout : [B, N, L, H, D]
* mask_bias     : [B, N, 1, 1, L]   additive, 0 or -1e9 per key
* pair_bias     : [B, 1, H, L, L]   additive, shared by every n

Rounding to the storage dtype is round-to-nearest-even: fp16 through NumPy's
own cast, bf16 by integer arithmetic on the float32 bit pattern.  -1e9 becomes
-inf in fp16 (it overflows) and -998244352 in bf16.

Draw order for one call (all float32, one ``numpy.random.default_rng(seed)``):
q, k, v ~ N(0,1); mask uniforms [B,N,L]; pair ~ N(0,1)*sigma (only when a
pair bias is requested); dout ~ N(0,1).  A key is masked where its uniform is
below ``mask_p`` or, for a padded batch, where it lies past its batch entry's
length.  If every key of one (b, n) row would be masked, key 0 is left
unmasked, so that no query row is fully masked.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional, Tuple

import numpy as np

MASK_VALUE = -1e9

DTYPES = ("fp16", "bf16")


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload: shape, dtype and input distribution."""

    name: str
    B: int
    N: int
    L: int
    H: int
    D: int
    dtype: str = "fp16"
    mask_p: Optional[float] = 0.05  # None: no mask bias at all
    pair_sigma: Optional[float] = 1.0  # None: no pair bias at all
    seed: int = 0
    # padded batch: keys j >= key_lengths[b] of every row of batch entry b are
    # masked (as a padded residue or sequence axis is); None: no padding
    key_lengths: Optional[Tuple[int, ...]] = None
    mask_value: float = MASK_VALUE  # the additive bias of a masked key

    @property
    def shape(self):
        return (self.B, self.N, self.L, self.H, self.D)

    @property
    def scores(self) -> int:
        return self.B * self.N * self.H * self.L * self.L

    @property
    def fwd_flops(self) -> int:
        # two GEMMs of B*N*H*L*L*D multiply-adds each
        return 4 * self.B * self.N * self.H * self.L * self.L * self.D


# The five workloads.  Shapes, dtypes and distributions are those of the
# evaluation configurations; the (1,256,256,4,32) and (1,512,256,8,8) shapes
# are also the unit-test shapes the DeepSpeed4Science guide lists (§3.5).
CONFIGS: Dict[str, Config] = {
    "tiny_row": Config("tiny_row", 1, 16, 32, 2, 8, "fp16", 0.10, 1.0, 1001),
    "msa_row": Config("msa_row", 1, 256, 256, 4, 32, "fp16", 0.05, 1.0, 1002),
    "msa_row_smalld": Config("msa_row_smalld", 1, 512, 256, 8, 8, "bf16", 0.05, 0.5, 1003),
    "msa_col": Config("msa_col", 1, 384, 512, 8, 32, "bf16", 0.10, None, 1004),
    "triangle": Config("triangle", 1, 768, 768, 4, 32, "bf16", 0.03, 1.0, 1005),
}
CONFIG_ORDER = ["tiny_row", "msa_row", "msa_row_smalld", "msa_col", "triangle"]


# ---------------------------------------------------------------- rounding


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u.astype(np.uint64) + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def from_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit pattern -> float64 values (exact)."""
    if dtype == "fp16":
        return f16_bits_to_f32(b).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(b).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------- generator


def make_inputs(cfg: Config, seed: Optional[int] = None) -> Dict[str, Optional[np.ndarray]]:
    """Draw one set of inputs; every tensor is returned as uint16 bits.

    Keys: q, k, v, mask_bias (or None), pair_bias (or None), dout.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, N, L, H, D = cfg.shape
    q = rng.standard_normal((B, N, L, H, D), dtype=np.float32)
    k = rng.standard_normal((B, N, L, H, D), dtype=np.float32)
    v = rng.standard_normal((B, N, L, H, D), dtype=np.float32)
    mask = None
    if cfg.mask_p is not None:
        u = rng.random((B, N, L), dtype=np.float32)
        masked = u < np.float32(cfg.mask_p)
        if cfg.key_lengths is not None:
            for b, n_keys in enumerate(cfg.key_lengths):
                masked[b, :, n_keys:] = True
        full = masked.all(axis=-1)
        masked[full, 0] = False
        mask = np.where(masked, np.float32(cfg.mask_value), np.float32(0.0)).astype(np.float32)
        mask = mask.reshape(B, N, 1, 1, L)
    pair = None
    if cfg.pair_sigma is not None:
        pair = rng.standard_normal((B, 1, H, L, L), dtype=np.float32) * np.float32(cfg.pair_sigma)
    dout = rng.standard_normal((B, N, L, H, D), dtype=np.float32)
    out = {
        "q": to_bits(q, cfg.dtype),
        "k": to_bits(k, cfg.dtype),
        "v": to_bits(v, cfg.dtype),
        "mask_bias": None if mask is None else to_bits(mask, cfg.dtype),
        "pair_bias": None if pair is None else to_bits(pair, cfg.dtype),
        "dout": to_bits(dout, cfg.dtype),
    }
    return out


def as_float64(bits: Dict[str, Optional[np.ndarray]], dtype: str) -> Dict[str, Optional[np.ndarray]]:
    return {k: (None if v is None else from_bits(v, dtype)) for k, v in bits.items()}


def digest(bits: Dict[str, Optional[np.ndarray]]) -> str:
    """sha256 over the tensors' bytes in a fixed key order (for logs)."""
    h = hashlib.sha256()
    for key in ("q", "k", "v", "mask_bias", "pair_bias", "dout"):
        a = bits.get(key)
        h.update(key.encode())
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def custom(name: str, B: int, N: int, L: int, H: int, D: int, dtype: str = "fp16",
           mask_p: Optional[float] = 0.1, pair_sigma: Optional[float] = 1.0, seed: int = 7,
           key_lengths: Optional[Tuple[int, ...]] = None, mask_value: float = MASK_VALUE) -> Config:
    if key_lengths is not None:
        assert len(key_lengths) == B and all(1 <= n <= L for n in key_lengths), key_lengths
    return Config(name, B, N, L, H, D, dtype, mask_p, pair_sigma, seed, key_lengths, mask_value)


# Padded batches of the MSA-row shape (1,256,256,4,32) fp16, keys past a
# length masked with -1e9 (which is -inf in fp16) on top of the 5% random key
# mask, same score count as the unpadded workload:
#  - uniform: one entry whose 160 residues are padded to 256 (62.5% of the
#    32-key blocks hold a live key; the rest are skipped by the kernels);
#  - mixed: four entries of 64 sequences with 256, 200, 160 and 96 residues
#    padded to 256 (72% live blocks, unevenly spread over the workgroups).
PADDED_UNIFORM = custom("msa_row_padded_uniform", 1, 256, 256, 4, 32, "fp16", 0.05, 1.0, 1013, key_lengths=(160,))
PADDED = custom("msa_row_padded_mixed", 4, 64, 256, 4, 32, "fp16", 0.05, 1.0, 1012, key_lengths=(256, 200, 160, 96))
