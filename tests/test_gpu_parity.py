"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Same seeded inputs on both sides (tests/helpers.py moves the generator's
bits to the GPU unchanged).  Tolerances are max-abs errors: fp16 5e-3 on
outputs and 2e-2 on gradients, bf16 2e-2 and 5e-2; lse 1e-3.  The bias
gradients are compared on their fp32 accumulators (read from the backward
workspace), and their dtype outputs must be exactly the round-to-nearest-even
cast of those accumulators.
"""
import sys

import numpy as np
import pytest
import torch

from evoformer_biased_attention_amd import inputs as I
from oracle import evo_oracle as O
from tests.helpers import LSE_TOL, TOL, bits_of, max_err, rne_bits, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run_gpu(cfg, bits):
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd, workspace_f32_views

    dt = cfg.dtype
    q, k, v = (to_device(bits[n], dt) for n in ("q", "k", "v"))
    m, p, do = to_device(bits["mask_bias"], dt), to_device(bits["pair_bias"], dt), to_device(bits["dout"], dt)
    out, lse = attn_fwd(q, k, v, m, p)
    g = attn_bwd(q, k, v, m, p, out, lse, do)
    torch.cuda.synchronize()
    delta, dmask32, dpair32 = workspace_f32_views(g["workspace"], cfg.shape, q.dtype, m is not None, p is not None)
    return {
        "out": out, "lse": lse, "dq": g["dq"], "dk": g["dk"], "dv": g["dv"], "dmask": g["dmask"], "dpair": g["dpair"],
        "dmask32": None if dmask32 is None else dmask32.clone(), "dpair32": None if dpair32 is None else dpair32.clone(),
        "delta": delta.clone(),
    }


def _compare(cfg, bits, res, ns=None, dpair_rows=None):
    x = I.as_float64(bits, cfg.dtype)
    tol = TOL[cfg.dtype]
    sel = slice(None) if ns is None else list(ns)
    o_ref, lse_ref = O.attention_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], ns=ns)
    g_ref = O.attention_bwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], x["dout"], ns=ns)
    errs = {}
    errs["out"] = max_err(to_f64(res["out"])[:, sel], o_ref)
    lse_gpu = to_f64(res["lse"])[:, sel]
    assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse_ref)), "lse -inf pattern differs"
    fin = np.isfinite(lse_ref)
    errs["lse"] = max_err(lse_gpu[fin], lse_ref[fin])
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
        else:
            ref_rows = O.dpair_rows(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], x["dout"], dpair_rows)
            got_rows = np.stack([d32[b, 0, h, i] for (b, h, i) in dpair_rows])
            errs["dpair32"] = max_err(got_rows, ref_rows)
        assert np.array_equal(bits_of(res["dpair"]), rne_bits(res["dpair32"].cpu().numpy(), cfg.dtype)), \
            "dpair output is not the RNE cast of its fp32 accumulator"
    print(f"  errors {cfg.name} {cfg.shape} {cfg.dtype}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    assert errs["out"] <= tol["out"], errs
    assert errs["lse"] <= LSE_TOL, errs
    assert errs["delta"] <= tol["grad"], errs
    for key in ("dq", "dk", "dv", "dmask32", "dpair32"):
        if key in errs:
            assert errs[key] <= tol["grad"], (key, errs)


SMALL = [
    I.custom("c1_tiny_row", 1, 16, 32, 2, 8, "fp16", 0.10, 1.0, 1001),
    I.custom("ragged100_d32", 1, 3, 100, 2, 32, "fp16", 0.1, 1.0, 11),
    I.custom("ragged77_d16_bf16", 2, 2, 77, 3, 16, "bf16", 0.1, 1.0, 12),
    I.custom("l200_d64", 1, 2, 200, 2, 64, "fp16", 0.1, 1.0, 13),
    I.custom("mask_only_d8_bf16", 1, 5, 33, 4, 8, "bf16", 0.2, None, 14),
    I.custom("pair_only_d32", 1, 3, 64, 2, 32, "fp16", None, 1.0, 15),
    I.custom("no_bias_d16_bf16", 1, 2, 48, 2, 16, "bf16", None, None, 16),
    I.custom("l1", 1, 3, 1, 2, 32, "fp16", None, 1.0, 17),
    I.custom("l17_d8", 2, 3, 17, 2, 8, "fp16", 0.2, 1.0, 18),
    I.custom("l300_streamed_pair_bf16", 1, 2, 300, 2, 32, "bf16", 0.05, 1.0, 19),
    I.custom("l520_d16", 1, 2, 520, 1, 16, "fp16", 0.05, 1.0, 20),
    I.custom("l800_atomic_dpair_bf16", 1, 2, 800, 1, 32, "bf16", 0.05, 1.0, 21),
    I.custom("n_odd_groups", 1, 37, 64, 2, 32, "bf16", 0.1, 1.0, 22),
    I.custom("pair_big_sigma", 1, 4, 96, 2, 32, "fp16", 0.1, 4.0, 23),
    # rows longer than one key tile: split query side, tiled key side
    I.custom("l600_no_bias", 1, 2, 600, 2, 32, "fp16", None, None, 24),
    I.custom("l384_mask_only_bf16", 1, 3, 384, 2, 16, "bf16", 0.1, None, 25),
    I.custom("l260_d64_gathered_bias", 1, 2, 260, 2, 64, "fp16", 0.1, 1.0, 26),
    I.custom("l513_d8_bf16", 1, 2, 513, 1, 8, "bf16", 0.05, 1.0, 27),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_parity_small_shapes(cfg):
    print(f"case {cfg.name} shape={cfg.shape} dtype={cfg.dtype} seed={cfg.seed}", flush=True)
    bits = I.make_inputs(cfg)
    res = _run_gpu(cfg, bits)
    _compare(cfg, bits, res)


@pytest.mark.parametrize("cfg", [SMALL[3], SMALL[-2]], ids=["l200_d64", "l260_d64"])
def test_parity_without_bias_gradients(cfg):
    """Only dQ, dK, dV requested: the kernels that skip the bias-gradient work."""
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd

    print(f"case no-bias-grads {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    bits = I.make_inputs(cfg)
    dt = cfg.dtype
    q, k, v = (to_device(bits[n], dt) for n in ("q", "k", "v"))
    m, p, do = to_device(bits["mask_bias"], dt), to_device(bits["pair_bias"], dt), to_device(bits["dout"], dt)
    out, lse = attn_fwd(q, k, v, m, p)
    g = attn_bwd(q, k, v, m, p, out, lse, do, want_dmask=False, want_dpair=False)
    torch.cuda.synchronize()
    assert g["dmask"] is None and g["dpair"] is None
    x = I.as_float64(bits, dt)
    g_ref = O.attention_bwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], x["dout"])
    tol = TOL[dt]["grad"]
    for key in ("dq", "dk", "dv"):
        err = max_err(to_f64(g[key]), g_ref[key])
        print(f"  {key} err {err:.2e}", flush=True)
        assert err <= tol, (key, err)


def _sample(n_total, k, seed):
    k = min(k, n_total)
    return sorted(np.random.default_rng(seed).choice(n_total, k, replace=False).tolist())


@pytest.mark.parametrize("name,n_slices,n_rows", [
    ("tiny_row", None, None),
    ("msa_row", None, None),
    ("msa_row_smalld", 16, 64),
    ("msa_col", 8, 0),
    ("triangle", 64, 64),
])
def test_parity_workloads(name, n_slices, n_rows):
    """The five workloads at full size; the large ones checked on sampled dim-1 slices
    (every output of those slices) and sampled dpair rows (summed over all n)."""
    cfg = I.CONFIGS[name]
    print(f"case {name} shape={cfg.shape} dtype={cfg.dtype} seed={cfg.seed}", flush=True)
    bits = I.make_inputs(cfg)
    res = _run_gpu(cfg, bits)
    if n_slices is None:
        _compare(cfg, bits, res)
    else:
        ns = _sample(cfg.N, n_slices, 1105)
        rows = None
        if cfg.pair_sigma is not None:
            rng = np.random.default_rng(1106)
            rows = [(0, int(rng.integers(cfg.H)), int(rng.integers(cfg.L))) for _ in range(n_rows)]
        _compare(cfg, bits, res, ns=ns, dpair_rows=rows)
