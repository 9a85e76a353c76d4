"""Blocks of keys masked with -inf: parity with the oracle where the kernels skip work.

A key whose mask bias is -inf has P = 0 in every row, so it adds nothing to O,
lse, dQ or dpair, and its dK, dV and dmask are zero.  The forward and the
query-side backward stop each key tile at its last key that is not -inf (the
32-key blocks past it are not computed), and a key-side backward wave whose 16
keys are all -inf skips the slice.  These cases put masked keys where those
paths run: padded batches (fp16, where -1e9 overflows to -inf, and bf16 with an
explicit -inf), whole key tiles past a row's padding, interior blocks of -inf
keys (computed, and exact either way), a whole slice with every key masked
(O = 0, lse = -inf, zero gradients), rows of one and of several key tiles,
D = 8, 16, 32 and 64, with and without the pair bias, -inf entries in the
pair bias itself, and batches whose entries the forward reorders by live length.
Tolerances and the comparison are those of the other parity tests.
"""
import numpy as np
import pytest

from evoformer_biased_attention_amd import inputs as I
from tests.helpers import compare_with_oracle as _compare, run_gpu as _run_gpu

pytestmark = pytest.mark.gpu

NEG_INF = float("-inf")

PADDED = [
    I.custom("pad_l256_d32", 2, 6, 256, 4, 32, "fp16", 0.05, 1.0, 41, key_lengths=(256, 97)),
    I.custom("pad_l200_d64", 2, 4, 200, 2, 64, "fp16", 0.05, 1.0, 42, key_lengths=(200, 50)),
    I.custom("pad_l520_d16", 2, 2, 520, 1, 16, "fp16", 0.05, 1.0, 43, key_lengths=(300, 520)),
    I.custom("pad_l384_bf16_inf_nopair", 2, 3, 384, 2, 32, "bf16", 0.05, None, 44, key_lengths=(384, 130),
             mask_value=NEG_INF),
    I.custom("pad_l256_bf16_inf", 2, 5, 256, 4, 32, "bf16", 0.05, 1.0, 45, key_lengths=(33, 256),
             mask_value=NEG_INF),
    I.custom("pad_l64_d8", 3, 4, 64, 2, 8, "fp16", 0.1, 1.0, 46, key_lengths=(64, 31, 1)),
]


@pytest.mark.parametrize("cfg", PADDED, ids=[c.name for c in PADDED])
def test_parity_padded_batches(cfg):
    print(f"case padded {cfg.name} shape={cfg.shape} dtype={cfg.dtype} lengths={cfg.key_lengths}", flush=True)
    bits = I.make_inputs(cfg)
    res = _run_gpu(cfg, bits)
    _compare(cfg, bits, res)


def _with_dead_blocks(cfg, blocks, dead_slices):
    """Inputs of cfg with keys [lo, hi) of every row masked to -inf for each (lo, hi)
    in blocks, and every key of the listed (b, n) slices masked to -inf."""
    bits = I.make_inputs(cfg)
    ninf = I.to_bits(np.array([NEG_INF], np.float32), cfg.dtype)[0]
    m = bits["mask_bias"].copy()
    for lo, hi in blocks:
        m[..., lo:hi] = ninf
    for b, n in dead_slices:
        m[b, n] = ninf
    bits["mask_bias"] = m
    return bits


DEAD = [
    (I.custom("dead_l256_d32", 1, 6, 256, 4, 32, "fp16", 0.05, 1.0, 51), [(32, 64), (160, 224)], [(0, 2)]),
    (I.custom("dead_l200_d64_bf16", 1, 4, 200, 2, 64, "bf16", 0.05, 1.0, 52), [(0, 32), (64, 128)], [(0, 3)]),
    (I.custom("dead_l600_d32", 1, 3, 600, 2, 32, "fp16", 0.05, 1.0, 53), [(256, 512)], [(0, 1)]),
    (I.custom("dead_l100_d16_nopair", 2, 3, 100, 2, 16, "fp16", 0.1, None, 54), [(0, 64)], [(1, 0)]),
]


@pytest.mark.parametrize("cfg,blocks,dead_slices", DEAD, ids=[c[0].name for c in DEAD])
def test_parity_interior_dead_blocks(cfg, blocks, dead_slices):
    print(f"case dead blocks {cfg.name} shape={cfg.shape} dtype={cfg.dtype} blocks={blocks} slices={dead_slices}",
          flush=True)
    bits = _with_dead_blocks(cfg, blocks, dead_slices)
    res = _run_gpu(cfg, bits)
    _compare(cfg, bits, res)
    # a slice with every key masked: O = 0, lse = -inf, zero gradients, exactly
    for b, n in dead_slices:
        for key in ("out", "dq", "dk", "dv"):
            assert not bool(res[key][b, n].any()), f"{key} of the fully masked slice is not zero"
        assert bool(np.isneginf(res["lse"][b, n].cpu().numpy()).all()), "lse of the fully masked slice"
        if res["dmask"] is not None:
            assert not bool(res["dmask"][b, n].any()), "dmask of the fully masked slice is not zero"


TRUNC = [
    (I.custom("trunc_l256_d32", 1, 3, 256, 2, 32, "fp16", 0.05, 1.0, 61), 150),
    (I.custom("trunc_l600_d16", 1, 2, 600, 1, 16, "fp16", 0.05, 1.0, 62), 300),
    (I.custom("trunc_l200_d64_bf16", 1, 2, 200, 2, 64, "bf16", 0.05, 1.0, 63, mask_value=NEG_INF), 77),
]


@pytest.mark.parametrize("cfg,n_keys", TRUNC, ids=[c[0].name for c in TRUNC])
def test_padding_equals_truncation(cfg, n_keys):
    """Keys past n_keys masked with -inf give, for the first n_keys queries, the same O, lse and dQ bits
    as the same problem cut to length n_keys (the padding is skipped, not computed as zeros)."""
    import torch

    print(f"case truncation {cfg.name} shape={cfg.shape} dtype={cfg.dtype} n_keys={n_keys}", flush=True)
    bits = I.make_inputs(cfg)
    ninf = I.to_bits(np.array([NEG_INF], np.float32), cfg.dtype)[0]
    bits["mask_bias"] = bits["mask_bias"].copy()
    bits["mask_bias"][..., n_keys:] = ninf
    n = n_keys
    cut = {
        "q": bits["q"][:, :, :n], "k": bits["k"][:, :, :n], "v": bits["v"][:, :, :n], "dout": bits["dout"][:, :, :n],
        "mask_bias": bits["mask_bias"][..., :n], "pair_bias": bits["pair_bias"][..., :n, :n],
    }
    B, N, L, H, D = cfg.shape
    cfg_cut = I.custom(cfg.name + "_cut", B, N, n, H, D, cfg.dtype, cfg.mask_p, cfg.pair_sigma, cfg.seed)
    full = _run_gpu(cfg, bits)
    short = _run_gpu(cfg_cut, cut)
    assert torch.equal(full["out"][:, :, :n], short["out"]), "O differs from the truncated problem"
    assert torch.equal(full["lse"][..., :n], short["lse"]), "lse differs from the truncated problem"
    assert torch.equal(full["dq"][:, :, :n], short["dq"]), "dQ differs from the truncated problem"
    # dpair sums over n in workgroup groups that depend on the row length: equal up to rounding
    d_full = full["dpair32"][:, :, :, :n, :n].double().cpu().numpy()
    d_short = short["dpair32"].double().cpu().numpy()
    assert np.max(np.abs(d_full - d_short)) <= 1e-4, "dpair differs from the truncated problem"


@pytest.mark.parametrize("cfg", [I.PADDED_UNIFORM, I.PADDED], ids=["padded_uniform", "padded_mixed"])
def test_parity_benchmark_padded_workloads(cfg):
    """The two padded workloads the benchmark times, at full size: every element of every
    output (dpair summed over all slices)."""
    print(f"case padded workload {cfg.name} shape={cfg.shape} dtype={cfg.dtype} lengths={cfg.key_lengths}",
          flush=True)
    bits = I.make_inputs(cfg)
    res = _run_gpu(cfg, bits)
    _compare(cfg, bits, res)


PAIR_INF = [
    I.custom("pinf_l72_d32_bf16_slab", 1, 3, 72, 2, 32, "bf16", 0.05, 1.0, 71),
    I.custom("pinf_l77_d16_bf16", 1, 2, 77, 2, 16, "bf16", 0.05, 1.0, 72),
    I.custom("pinf_l300_d32_bf16_streamed", 1, 2, 300, 2, 32, "bf16", 0.05, 1.0, 73),
    I.custom("pinf_l96_d64_bf16", 1, 2, 96, 2, 64, "bf16", None, 1.0, 74),
    I.custom("pinf_l40_d8_bf16", 1, 3, 40, 2, 8, "bf16", 0.1, 1.0, 75),
    I.custom("pinf_l100_d32_fp16", 1, 3, 100, 2, 32, "fp16", 0.05, 1.0, 76),
    # rows longer than one key tile with vector bias loads: the forward's bias
    # ring and bwd_kv3's per-wave bias regions (bf16 and fp16)
    I.custom("pinf_l320_d32_bf16_streamed_vec", 1, 2, 320, 2, 32, "bf16", 0.05, 1.0, 77),
    I.custom("pinf_l264_d32_fp16_streamed", 1, 2, 264, 2, 32, "fp16", 0.05, 1.0, 78),
]


@pytest.mark.parametrize("cfg", PAIR_INF, ids=[c.name for c in PAIR_INF])
def test_parity_pair_bias_neg_inf(cfg):
    """-inf entries in the pair bias: 5% of them at seeded positions, one query row
    of head 0 entirely (that row of every slice has O = 0, lse = -inf and zero
    dQ) and one key column of head 1 entirely.  Such a score is -inf, as with the
    mask: P = 0 there, no NaN anywhere (bf16 adds the pair bias through the MFMA,
    whose zeros off the diagonal meet it), and the gradients are the oracle's."""
    print(f"case pair -inf {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    bits = I.make_inputs(cfg)
    B, N, L, H, D = cfg.shape
    ninf = I.to_bits(np.array([NEG_INF], np.float32), cfg.dtype)[0]
    p = bits["pair_bias"].copy()
    rng = np.random.default_rng(cfg.seed)
    p[rng.random(p.shape) < 0.05] = ninf
    i_dead, j_dead = min(3, L - 1), min(5, L - 1)
    p[:, 0, 0, i_dead, :] = ninf
    p[:, 0, 1, :, j_dead] = ninf
    bits["pair_bias"] = p
    res = _run_gpu(cfg, bits)
    for key in ("out", "lse", "dq", "dk", "dv"):
        assert not bool(res[key].isnan().any()), f"NaN in {key}"
    _compare(cfg, bits, res)
    assert not bool(res["out"][:, :, i_dead, 0].any()), "O of the query row with every pair entry -inf"
    assert bool(np.isneginf(res["lse"][:, :, 0, i_dead].cpu().numpy()).all()), "lse of that row"
    assert not bool(res["dq"][:, :, i_dead, 0].any()), "dQ of that row"
    assert not bool(res["dk"][:, :, j_dead, 1].any()) and not bool(res["dv"][:, :, j_dead, 1].any()), \
        "dK, dV of the key with every pair entry -inf"


BALANCED = [
    I.custom("balanced_fp16_unsorted", 4, 64, 256, 4, 32, "fp16", 0.05, 1.0, 81, key_lengths=(96, 256, 160, 200)),
    I.custom("balanced_bf16_inf_unsorted", 4, 64, 256, 4, 32, "bf16", 0.05, 1.0, 82, key_lengths=(200, 64, 256, 130),
             mask_value=NEG_INF),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", BALANCED, ids=[c.name for c in BALANCED])
def test_parity_balanced_forward_order(cfg):
    """Batch entries of different live lengths, in an order that is not sorted by
    length, at a size whose forward grid is one round of two workgroups per CU:
    the forward takes the entries in the order of their live blocks, pairing long
    with short work on each CU.  Every element of every output against the oracle."""
    print(f"case balanced order {cfg.name} shape={cfg.shape} dtype={cfg.dtype} lengths={cfg.key_lengths}",
          flush=True)
    bits = I.make_inputs(cfg)
    res = _run_gpu(cfg, bits)
    _compare(cfg, bits, res)
