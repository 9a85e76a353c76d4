"""The seeded input generator: determinism, rounding and the mask rule."""
import json
import os

import numpy as np
import torch

from evoformer_biased_attention_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e9, -1e9, 65504.0, 3.0e38, -3.0e38, 1e-40], dtype=np.float32)])
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = I.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_mask_value_in_each_dtype():
    f16 = I.from_bits(I.to_bits(np.array([-1e9], np.float32), "fp16"), "fp16")[0]
    bf16 = I.from_bits(I.to_bits(np.array([-1e9], np.float32), "bf16"), "bf16")[0]
    assert np.isneginf(f16)
    assert bf16 == -998244352.0


def test_every_row_keeps_an_unmasked_key():
    cfg = I.custom("allmask", 2, 50, 3, 1, 8, "fp16", mask_p=0.97, seed=3)
    x = I.as_float64(I.make_inputs(cfg), "fp16")
    m = x["mask_bias"][:, :, 0, 0, :]
    assert np.all((m == 0).any(axis=-1))
    assert np.isneginf(m).any()


def test_deterministic_and_matches_golden_digest():
    with open(os.path.join(GOLDEN, "input_digests.json")) as f:
        gold = json.load(f)
    for name in ("tiny_row",):
        cfg = I.CONFIGS[name]
        a = I.make_inputs(cfg)
        b = I.make_inputs(cfg)
        assert I.digest(a) == I.digest(b) == gold[name]


def test_config_shapes_and_fractions():
    cfg = I.CONFIGS["msa_row"]
    x = I.make_inputs(cfg)
    assert x["q"].shape == (1, 256, 256, 4, 32) and x["q"].dtype == np.uint16
    assert x["mask_bias"].shape == (1, 256, 1, 1, 256)
    assert x["pair_bias"].shape == (1, 1, 4, 256, 256)
    frac = np.isneginf(I.from_bits(x["mask_bias"], "fp16")).mean()
    assert 0.04 < frac < 0.06
    assert I.CONFIGS["msa_col"].pair_sigma is None
    assert I.make_inputs(I.custom("np", 1, 2, 4, 1, 8, pair_sigma=None))["pair_bias"] is None


def test_padded_batches_mask_past_each_length():
    """Keys at or past an entry's length are masked in every row of it; the keys before keep the random
    mask of the same seed without padding (the padding draws nothing)."""
    for cfg in (I.PADDED, I.PADDED_UNIFORM):
        x = I.as_float64(I.make_inputs(cfg), cfg.dtype)["mask_bias"][:, :, 0, 0, :]
        for b, n_keys in enumerate(cfg.key_lengths):
            assert np.isneginf(x[b, :, n_keys:]).all()
            assert (x[b, :, :n_keys] == 0).mean() > 0.9
    cfg = I.custom("p", 2, 3, 40, 1, 8, "bf16", 0.1, None, 5, key_lengths=(40, 9), mask_value=float("-inf"))
    plain = I.custom("p", 2, 3, 40, 1, 8, "bf16", 0.1, None, 5, mask_value=float("-inf"))
    a = I.as_float64(I.make_inputs(cfg), "bf16")
    p = I.as_float64(I.make_inputs(plain), "bf16")
    assert np.isneginf(a["mask_bias"][1, :, 0, 0, 9:]).all()
    assert np.array_equal(a["mask_bias"][0], p["mask_bias"][0])
    assert np.array_equal(a["mask_bias"][1, :, :, :, :9], p["mask_bias"][1, :, :, :, :9])
    for key in ("q", "k", "v", "dout"):
        assert np.array_equal(a[key], p[key])
