"""Shared test helpers: seeded inputs onto the GPU, oracle comparison.

Nothing here computes attention: the GPU side calls the C ABI through the
package binding, the expected side calls oracle/ only.
"""
from __future__ import annotations

import numpy as np
import torch

from evoformer_biased_attention_amd import inputs as I
from oracle import evo_oracle as O

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


def run_gpu(cfg, bits, partial_budget=None):
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd, workspace_f32_views

    dt = cfg.dtype
    q, k, v = (to_device(bits[n], dt) for n in ("q", "k", "v"))
    m, p, do = to_device(bits["mask_bias"], dt), to_device(bits["pair_bias"], dt), to_device(bits["dout"], dt)
    out, lse = attn_fwd(q, k, v, m, p)
    g = attn_bwd(q, k, v, m, p, out, lse, do, partial_budget=partial_budget)
    torch.cuda.synchronize()
    delta, dmask32, dpair32 = workspace_f32_views(g["workspace"], cfg.shape, q.dtype, m is not None, p is not None)
    return {
        "out": out, "lse": lse, "dq": g["dq"], "dk": g["dk"], "dv": g["dv"], "dmask": g["dmask"], "dpair": g["dpair"],
        "dmask32": None if dmask32 is None else dmask32.clone(), "dpair32": None if dpair32 is None else dpair32.clone(),
        "delta": delta.clone(),
    }


def compare_with_oracle(cfg, bits, res, ns=None, dpair_rows=None, parts=("fwd", "bwd")):
    """Every output in ``res`` against the oracle on the same input bits.

    ``ns``: compare only these dim-1 slices (None: all).  dpair sums over every
    slice, so with ``ns`` it is compared on ``dpair_rows`` (b, h, i), each summed
    over all n by the oracle, or not at all when that is None.  ``parts``
    selects the forward outputs (O, lse), the backward ones (delta, dQ, dK, dV,
    dmask, dpair) or both.
    """
    x = I.as_float64(bits, cfg.dtype)
    tol = TOL[cfg.dtype]
    sel = slice(None) if ns is None else list(ns)
    errs = {}
    if "fwd" in parts:
        o_ref, lse_ref = O.attention_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], ns=ns)
        errs["out"] = max_err(to_f64(res["out"])[:, sel], o_ref)
        lse_gpu = to_f64(res["lse"])[:, sel]
        assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse_ref)), "lse -inf pattern differs"
        fin = np.isfinite(lse_ref)
        errs["lse"] = max_err(lse_gpu[fin], lse_ref[fin])
        del o_ref, lse_ref
    if "bwd" in parts:
        g_ref = O.attention_bwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], x["dout"], ns=ns)
        for key in ("dq", "dk", "dv"):
            errs[key] = max_err(to_f64(res[key])[:, sel], g_ref[key])
        errs["delta"] = max_err(to_f64(res["delta"])[:, sel], g_ref["delta"])
        if res["dmask"] is not None:
            errs["dmask32"] = max_err(to_f64(res["dmask32"])[:, sel], g_ref["dmask"])
            assert np.array_equal(bits_of(res["dmask"]), rne_bits(res["dmask32"].cpu().numpy(), cfg.dtype)), \
                "dmask output is not the RNE cast of its fp32 accumulator"
        if res["dpair"] is not None:
            d32 = to_f64(res["dpair32"])
            if ns is None:
                errs["dpair32"] = max_err(d32, g_ref["dpair"])
            elif dpair_rows is not None:
                ref_rows = O.dpair_rows(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], x["dout"], dpair_rows)
                got_rows = np.stack([d32[b, 0, h, i] for (b, h, i) in dpair_rows])
                errs["dpair32"] = max_err(got_rows, ref_rows)
            assert np.array_equal(bits_of(res["dpair"]), rne_bits(res["dpair32"].cpu().numpy(), cfg.dtype)), \
                "dpair output is not the RNE cast of its fp32 accumulator"
    print(f"  errors {cfg.name} {cfg.shape} {cfg.dtype}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    if "out" in errs:
        assert errs["out"] <= tol["out"], errs
        assert errs["lse"] <= LSE_TOL, errs
    if "delta" in errs:
        assert errs["delta"] <= tol["grad"], errs
    for key in ("dq", "dk", "dv", "dmask32", "dpair32"):
        if key in errs:
            assert errs[key] <= tol["grad"], (key, errs)
    return errs
