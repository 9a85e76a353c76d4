"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Same seeded inputs on both sides (tests/helpers.py moves the generator's
bits to the GPU unchanged).  Tolerances are max-abs errors: fp16 5e-3 on
outputs and 2e-2 on gradients, bf16 2e-2 and 5e-2; lse 1e-3.  The bias
gradients are compared on their fp32 accumulators (read from the backward
workspace), and their dtype outputs must be exactly the round-to-nearest-even
cast of those accumulators.
"""
import numpy as np
import pytest
import torch

from evoformer_biased_attention_amd import inputs as I
from oracle import evo_oracle as O
from tests.helpers import TOL, compare_with_oracle, max_err, run_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu


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
    # bf16 pair bias on rows longer than one key tile, L % 8 == 0 (vector bias
    # loads: the forward's bias ring, the key side's bias regions) at D = 8, 16
    I.custom("l320_d8_bf16_pair", 1, 2, 320, 2, 8, "bf16", 0.05, 1.0, 28),
    I.custom("l264_d16_bf16_pair", 1, 3, 264, 1, 16, "bf16", 0.05, 1.0, 29),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_parity_small_shapes(cfg):
    print(f"case {cfg.name} shape={cfg.shape} dtype={cfg.dtype} seed={cfg.seed}", flush=True)
    bits = I.make_inputs(cfg)
    res = run_gpu(cfg, bits)
    compare_with_oracle(cfg, bits, res)


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


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny_row", "msa_row", "msa_row_smalld", "msa_col"])
def test_parity_workloads_full(name):
    """Four of the five workloads at full size, every element of every output
    (dpair summed over all n) against the oracle."""
    cfg = I.CONFIGS[name]
    print(f"case {name} shape={cfg.shape} dtype={cfg.dtype} seed={cfg.seed} (all slices)", flush=True)
    bits = I.make_inputs(cfg)
    res = run_gpu(cfg, bits)
    compare_with_oracle(cfg, bits, res)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", ["fwd", "bwd"])
def test_parity_triangle_full(part):
    """The triangle workload (1,768,768,4,32) bf16 at full size: every element of
    O and lse (part fwd), or of delta, dQ, dK, dV, dmask and dpair, the latter
    summed over all 768 slices by a streamed oracle pass (part bwd)."""
    cfg = I.CONFIGS["triangle"]
    print(f"case triangle {part} shape={cfg.shape} dtype={cfg.dtype} seed={cfg.seed} (all slices)", flush=True)
    bits = I.make_inputs(cfg)
    res = run_gpu(cfg, bits)
    compare_with_oracle(cfg, bits, res, parts=(part,))


# rows longer than one key tile with a pair bias run with partial budgets
# below what their fp32 partials take at once: bwd_q3 then goes over chunks of
# slices (the last one ragged) and the dpair slots carry their sums from chunk
# to chunk (rows without a pair bias keep dQ in registers and never chunk)
CHUNKED = [
    I.custom("chunked_b2_l640_d64_bf16", 2, 48, 640, 2, 64, "bf16", 0.05, 1.0, 31),
    I.custom("chunked_l520_fp16", 1, 120, 520, 4, 32, "fp16", 0.1, 1.0, 32),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", CHUNKED, ids=[c.name for c in CHUNKED])
def test_parity_long_rows_in_chunks(cfg):
    from evoformer_biased_attention_amd import _lib

    print(f"case chunked {cfg.name} shape={cfg.shape} dtype={cfg.dtype} seed={cfg.seed}", flush=True)
    B, N, L, H, D = cfg.shape
    jtiles = -(-L // (128 if D == 64 else 256))
    dt = {"fp16": _lib.EVO_F16, "bf16": _lib.EVO_BF16}[cfg.dtype]
    bits = I.make_inputs(cfg)
    ref = run_gpu(cfg, bits)  # the default plan
    compare_with_oracle(cfg, bits, ref)
    for budget in (96 << 20, 24 << 20):
        ws = _lib.evo_attn_bwd_workspace_bytes_within(cfg.shape, dt, cfg.mask_p is not None,
                                                      cfg.pair_sigma is not None, budget)
        assert ws < jtiles * B * N * L * H * D * 4, "the plan was expected to go in chunks"
        print(f"  partial budget {budget >> 20} MiB: workspace {ws / 1e6:.1f} MB", flush=True)
        res = run_gpu(cfg, bits, partial_budget=budget)
        # dQ keeps its key-tile order and dK, dV, dmask come from the same
        # kernels: the same bits; only dpair's summation order changes
        for n in ("out", "lse", "delta", "dq", "dk", "dv", "dmask", "dmask32"):
            if ref[n] is not None:
                assert torch.equal(res[n], ref[n]), n
        compare_with_oracle(cfg, bits, res, parts=("bwd",))


INFER = [SMALL[0], SMALL[1], SMALL[2], SMALL[3], SMALL[9], SMALL[10], SMALL[16], I.CONFIGS["msa_row"],
         I.CONFIGS["msa_row_smalld"]]


@pytest.mark.parametrize("cfg", INFER, ids=[c.name for c in INFER])
def test_inference_forward_against_oracle(cfg):
    """The forward that keeps no lse (guide §3.2: the forward kernels serve
    inference for every attention type): its output against the oracle's O,
    through the C ABI with lse = NULL and through evoformer_attention with no
    gradient."""
    from evoformer_biased_attention_amd import _lib
    from evoformer_biased_attention_amd.attention import attn_fwd, evoformer_attention

    print(f"case inference fwd vs oracle {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    bits = I.make_inputs(cfg)
    dt = cfg.dtype
    q, k, v = (to_device(bits[n], dt) for n in ("q", "k", "v"))
    m, p = to_device(bits["mask_bias"], dt), to_device(bits["pair_bias"], dt)
    out = torch.empty_like(q)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = _lib.evo_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), ptr(m), ptr(p), out.data_ptr(), None,
                           cfg.shape, {"fp16": _lib.EVO_F16, "bf16": _lib.EVO_BF16}[dt],
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    with torch.no_grad():
        out2 = evoformer_attention(q, k, v, [m, p])
    out3, none = attn_fwd(q, k, v, m, p, need_lse=False)
    torch.cuda.synchronize()
    assert none is None
    x = I.as_float64(bits, dt)
    o_ref, _ = O.attention_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"])
    tol = TOL[dt]["out"]
    for name, t in (("c_abi", out), ("evoformer_attention", out2), ("attn_fwd", out3)):
        err = max_err(to_f64(t), o_ref)
        print(f"  {name} out err {err:.2e}", flush=True)
        assert err <= tol, (name, err)
