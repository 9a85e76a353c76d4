"""Pins for the fp64 CPU oracle, checked against facts that do not come from it.

Each test names what fixes the expected value: a closed form, a library
routine (torch's scaled-dot-product attention in float64 on the CPU, scipy's
softmax), central finite differences, an algebraic identity, an invariance,
or a hand-derived worked example stored under tests/golden/.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import evo_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, B, N, L, H, D, mask_p=0.3, mask_val=-3.0, pair=True, mask=True):
    q = rng.standard_normal((B, N, L, H, D))
    k = rng.standard_normal((B, N, L, H, D))
    v = rng.standard_normal((B, N, L, H, D))
    do = rng.standard_normal((B, N, L, H, D))
    b1 = None
    if mask:
        u = rng.random((B, N, 1, 1, L))
        b1 = np.where(u < mask_p, mask_val, 0.0) + 0.1 * rng.standard_normal((B, N, 1, 1, L))
    b2 = rng.standard_normal((B, 1, H, L, L)) if pair else None
    return q, k, v, b1, b2, do


# ------------------------------------------------------------ closed forms


def test_worked_example_hand_derived():
    """A 1x2 problem whose answer is derived by hand (tests/golden/worked_example.json)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=np.float64)
    k = np.array(ex["k"], dtype=np.float64)
    v = np.array(ex["v"], dtype=np.float64)
    b1 = np.array(ex["mask_bias"], dtype=np.float64)
    b2 = np.array(ex["pair_bias"], dtype=np.float64)
    do = np.array(ex["dout"], dtype=np.float64)
    out, lse = O.attention_fwd(q, k, v, b1, b2)
    np.testing.assert_allclose(out.ravel(), ex["expect_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.ravel(), ex["expect_lse"], rtol=0, atol=1e-12)
    g = O.attention_bwd(q, k, v, b1, b2, do)
    np.testing.assert_allclose(g["dv"].ravel(), ex["expect_dv"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dmask"].ravel(), ex["expect_dmask"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dpair"].ravel(), ex["expect_dpair"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dq"].ravel(), ex["expect_dq"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk"].ravel(), ex["expect_dk"], rtol=0, atol=1e-12)


def test_rows_of_p_sum_to_one():
    rng = np.random.default_rng(1)
    q, k, v, b1, b2, _ = _rand(rng, 1, 3, 11, 2, 4, mask_val=-1e9)
    for n in range(3):
        _, _, p = O.slice_forward(q[0, n], k[0, n], v[0, n], b1[0, n, 0, 0], b2[0, 0])
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-12


def test_q_zero_gives_bias_softmax_mean_of_v():
    """Q = 0: scores reduce to the biases, O = softmax_j(b1 + b2) V whatever K is."""
    rng = np.random.default_rng(2)
    q, k, v, b1, b2, _ = _rand(rng, 2, 3, 9, 2, 5)
    q[:] = 0.0
    out, _ = O.attention_fwd(q, k, v, b1, b2)
    for b in range(2):
        for n in range(3):
            for h in range(2):
                w = scipy.special.softmax(b1[b, n, 0, 0][None, :] + b2[b, 0, h], axis=-1)
                ref = w @ v[b, n, :, h, :]
                np.testing.assert_allclose(out[b, n, :, h, :], ref, rtol=0, atol=1e-13)


def test_textbook_attention_when_n_h_one_without_bias():
    rng = np.random.default_rng(3)
    L, D = 13, 6
    q, k, v, _, _, _ = _rand(rng, 1, 1, L, 1, D, pair=False, mask=False)
    out, lse = O.attention_fwd(q, k, v, None, None)
    Q, K, V = q[0, 0, :, 0], k[0, 0, :, 0], v[0, 0, :, 0]
    s = Q @ K.T / np.sqrt(D)
    ref = scipy.special.softmax(s, axis=-1) @ V
    np.testing.assert_allclose(out[0, 0, :, 0], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0, 0], scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-13)


# ------------------------------------------------------ library routine pin


@pytest.mark.parametrize("shape", [(1, 3, 7, 2, 4), (2, 2, 10, 3, 8), (1, 4, 5, 1, 3)])
@pytest.mark.parametrize("with_mask,with_pair", [(True, True), (True, False), (False, True)])
def test_matches_torch_sdpa_float64(shape, with_mask, with_pair):
    """torch's scaled_dot_product_attention (CPU, float64, autograd) as an independent library pin.

    The biases enter as one additive float mask b1 + b2 broadcast to
    [B,N,H,L,L]; autograd sums their gradients over the broadcast dims.
    """
    rng = np.random.default_rng(sum(shape) + 10 * with_mask + with_pair)
    q, k, v, b1, b2, do = _rand(rng, *shape, mask=with_mask, pair=with_pair, mask_val=-1e9)
    out, lse = O.attention_fwd(q, k, v, b1, b2)
    g = O.attention_bwd(q, k, v, b1, b2, do)

    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv = T(q), T(k), T(v)
    tb1 = T(b1) if b1 is not None else None
    tb2 = T(b2) if b2 is not None else None
    perm = lambda t: t.permute(0, 1, 3, 2, 4)  # [B,N,H,L,D]
    bias = None
    if tb1 is not None:
        bias = tb1
    if tb2 is not None:
        bias = tb2 if bias is None else bias + tb2
    B, N, L, H, D = shape
    bias_full = bias.expand(B, N, H, L, L)
    ref = torch.nn.functional.scaled_dot_product_attention(perm(tq), perm(tk), perm(tv), attn_mask=bias_full)
    ref = ref.permute(0, 1, 3, 2, 4)
    np.testing.assert_allclose(out, ref.detach().numpy(), rtol=0, atol=1e-12)
    s = torch.matmul(perm(tq), perm(tk).transpose(-1, -2)) / np.sqrt(D) + bias_full
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).detach().numpy(), rtol=0, atol=1e-10)
    ref.backward(torch.tensor(do))
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), rtol=0, atol=1e-12)
    if tb1 is not None:
        np.testing.assert_allclose(g["dmask"], tb1.grad.numpy(), rtol=0, atol=1e-12)
    if tb2 is not None:
        np.testing.assert_allclose(g["dpair"], tb2.grad.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------ finite differences


@pytest.mark.parametrize("shape", [(1, 2, 5, 2, 3), (1, 3, 7, 2, 4)])
def test_finite_differences_every_element(shape):
    """Central differences (h = 1e-6) of sum(O * dO) w.r.t. every input element.

    The mask is finite (-3.0) so that its gradient flows.
    """
    rng = np.random.default_rng(shape[2])
    q, k, v, b1, b2, do = _rand(rng, *shape, mask_val=-3.0)
    g = O.attention_bwd(q, k, v, b1, b2, do)

    def loss(q_, k_, v_, b1_, b2_):
        o, _ = O.attention_fwd(q_, k_, v_, b1_, b2_)
        return float((o * do).sum())

    h = 1e-6
    args = {"q": q, "k": k, "v": v, "b1": b1, "b2": b2}
    grads = {"q": g["dq"], "k": g["dk"], "v": g["dv"], "b1": g["dmask"], "b2": g["dpair"]}
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a_p = {kk: vv.copy() for kk, vv in args.items()}
            a_m = {kk: vv.copy() for kk, vv in args.items()}
            a_p[name][idx] += h
            a_m[name][idx] -= h
            fd[idx] = (loss(a_p["q"], a_p["k"], a_p["v"], a_p["b1"], a_p["b2"])
                       - loss(a_m["q"], a_m["k"], a_m["v"], a_m["b1"], a_m["b2"])) / (2 * h)
        err = np.max(np.abs(fd - grads[name])) / max(1.0, np.max(np.abs(fd)))
        assert err <= 1e-6, (name, err)


# ---------------------------------------------------------- masked keys


def test_masked_keys_contribute_exactly_zero():
    """Keys with bias -inf (fp16's -1e9) or -1e9 (bf16's) carry zero weight exactly."""
    rng = np.random.default_rng(5)
    for mask_val in (-np.inf, -998244352.0):
        q, k, v, b1, b2, do = _rand(rng, 1, 3, 12, 2, 4, mask_p=0.3, mask_val=0.0)
        masked = rng.random((1, 3, 1, 1, 12)) < 0.3
        masked[..., 0] = False
        b1 = np.where(masked, mask_val, b1)
        out, lse = O.attention_fwd(q, k, v, b1, b2)
        g = O.attention_bwd(q, k, v, b1, b2, do)
        k2, v2 = k.copy(), v.copy()
        mk = masked[:, :, 0, 0, :]  # [B,N,L]
        k2[mk] = rng.standard_normal(k2[mk].shape) * 100
        v2[mk] = rng.standard_normal(v2[mk].shape) * 100
        out2, lse2 = O.attention_fwd(q, k2, v2, b1, b2)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
        assert np.all(g["dk"][mk] == 0.0) and np.all(g["dv"][mk] == 0.0)
        assert np.all(g["dmask"][masked] == 0.0)


def test_fully_masked_row_convention():
    rng = np.random.default_rng(6)
    q, k, v, b1, b2, do = _rand(rng, 1, 2, 6, 2, 4)
    b1[0, 1] = -np.inf
    out, lse = O.attention_fwd(q, k, v, b1, b2)
    g = O.attention_bwd(q, k, v, b1, b2, do)
    assert np.all(out[0, 1] == 0) and np.all(np.isneginf(lse[0, 1]))
    for key in ("dq", "dk", "dv"):
        assert np.all(g[key][0, 1] == 0)
    assert np.all(np.isfinite(out[0, 0])) and np.all(np.isfinite(g["dpair"]))


# ------------------------------------------------- identities, invariances


def test_gradient_identities():
    rng = np.random.default_rng(7)
    q, k, v, b1, b2, do = _rand(rng, 2, 3, 9, 2, 5)
    g = O.attention_bwd(q, k, v, b1, b2, do)
    assert np.max(np.abs(g["dpair"].sum(-1))) <= 1e-10
    assert np.max(np.abs(g["dmask"].sum(-1))) <= 1e-10
    for b in range(2):
        for n in range(3):
            for h in range(2):
                qq = (q[b, n, :, h] * g["dq"][b, n, :, h]).sum()
                kk = (k[b, n, :, h] * g["dk"][b, n, :, h]).sum()
                assert abs(qq - kk) <= 1e-10
                vv = (v[b, n, :, h] * g["dv"][b, n, :, h]).sum()
                assert abs(vv - g["delta"][b, n, h].sum()) <= 1e-10
    # delta from the chain rule equals rowsum(dO * O), the form a fused kernel uses
    out, _ = O.attention_fwd(q, k, v, b1, b2)
    np.testing.assert_allclose(g["delta"], (do * out).sum(-1).transpose(0, 1, 3, 2), rtol=0, atol=1e-12)


def test_invariances():
    rng = np.random.default_rng(8)
    q, k, v, b1, b2, do = _rand(rng, 1, 2, 8, 2, 4)
    out, lse = O.attention_fwd(q, k, v, b1, b2)
    # shifting one row's mask bias by c shifts lse by c and leaves O
    c = 3.25
    b1s = b1.copy()
    b1s[0, 1] += c
    out_s, lse_s = O.attention_fwd(q, k, v, b1s, b2)
    np.testing.assert_allclose(out_s, out, atol=1e-13)
    np.testing.assert_allclose(lse_s[0, 1], lse[0, 1] + c, atol=1e-12)
    np.testing.assert_allclose(lse_s[0, 0], lse[0, 0], atol=0)
    # permuting keys jointly (K, V, mask and pair columns) leaves O
    perm = rng.permutation(8)
    out_p, lse_p = O.attention_fwd(q, k[:, :, perm], v[:, :, perm], b1[..., perm], b2[..., perm])
    np.testing.assert_allclose(out_p, out, atol=1e-13)
    np.testing.assert_allclose(lse_p, lse, atol=1e-13)
    # linear in V
    v2 = rng.standard_normal(v.shape)
    o2, _ = O.attention_fwd(q, k, v2, b1, b2)
    o3, _ = O.attention_fwd(q, k, 2.0 * v - 0.5 * v2, b1, b2)
    np.testing.assert_allclose(o3, 2.0 * out - 0.5 * o2, atol=1e-12)


def test_identical_slices_scale_dpair():
    rng = np.random.default_rng(9)
    q, k, v, b1, b2, do = _rand(rng, 1, 1, 7, 2, 3)
    g1 = O.attention_bwd(q, k, v, b1, b2, do)
    rep = lambda a: np.repeat(a, 4, axis=1)
    g4 = O.attention_bwd(rep(q), rep(k), rep(v), rep(b1), b2, rep(do))
    np.testing.assert_allclose(g4["dpair"], 4.0 * g1["dpair"], atol=1e-12)


def test_dpair_rows_matches_full_backward():
    rng = np.random.default_rng(10)
    q, k, v, b1, b2, do = _rand(rng, 2, 3, 9, 2, 4, mask_val=-1e9)
    g = O.attention_bwd(q, k, v, b1, b2, do)
    rows = [(0, 0, 0), (1, 1, 8), (0, 1, 4), (1, 0, 3)]
    r = O.dpair_rows(q, k, v, b1, b2, do, rows)
    for t, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(r[t], g["dpair"][b, 0, h, i], atol=1e-12)


def test_sampled_slices_equal_full():
    rng = np.random.default_rng(11)
    q, k, v, b1, b2, do = _rand(rng, 1, 5, 6, 2, 4)
    full_o, full_l = O.attention_fwd(q, k, v, b1, b2)
    ns = [4, 1]
    o, l = O.attention_fwd(q, k, v, b1, b2, ns=ns)
    assert np.array_equal(o, full_o[:, ns]) and np.array_equal(l, full_l[:, ns])
    g = O.attention_bwd(q, k, v, b1, b2, do)
    gs = O.attention_bwd(q, k, v, b1, b2, do, ns=ns)
    for key in ("dq", "dk", "dv", "dmask"):
        assert np.array_equal(gs[key], g[key][:, ns])
    assert gs["dpair"] is None


# ------------------------------------------- planted mistakes are caught


def _sdpa_max_err(seed=21):
    rng = np.random.default_rng(seed)
    shape = (1, 2, 6, 2, 4)
    q, k, v, b1, b2, do = _rand(rng, *shape, mask_val=-2.0)
    out, _ = O.attention_fwd(q, k, v, b1, b2)
    g = O.attention_bwd(q, k, v, b1, b2, do)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tb1, tb2 = T(q), T(k), T(v), T(b1), T(b2)
    perm = lambda t: t.permute(0, 1, 3, 2, 4)
    B, N, L, H, D = shape
    ref = torch.nn.functional.scaled_dot_product_attention(
        perm(tq), perm(tk), perm(tv), attn_mask=(tb1 + tb2).expand(B, N, H, L, L)).permute(0, 1, 3, 2, 4)
    ref.backward(torch.tensor(do))
    errs = [np.abs(out - ref.detach().numpy()).max()]
    for key, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dmask", tb1), ("dpair", tb2)):
        errs.append(np.abs(g[key] - t.grad.numpy()).max())
    return max(errs)


def test_planted_mistakes_fail_the_library_pin(monkeypatch):
    """Each plausible slip in the oracle (on the CPU) moves it away from torch's SDPA."""
    assert _sdpa_max_err() < 1e-12
    orig_scores = O._slice_scores
    orig_backward = O.slice_backward
    mutations = {
        "scale 1/D": lambda: monkeypatch.setattr(O, "_scale", lambda D: 1.0 / D),
        "pair transposed": lambda: monkeypatch.setattr(
            O, "_slice_scores", lambda qs, ks, b1, b2, sc: orig_scores(qs, ks, b1, b2.transpose(0, 2, 1), sc)),
        "bias scaled": lambda: monkeypatch.setattr(
            O, "_slice_scores", lambda qs, ks, b1, b2, sc: orig_scores(qs, ks, b1 * sc, b2 * sc, sc)),
        "dK sign": lambda: monkeypatch.setattr(
            O, "slice_backward", lambda *a: {**orig_backward(*a), "dk": -orig_backward(*a)["dk"]}),
        "dpair misses delta": lambda: monkeypatch.setattr(
            O, "slice_backward",
            lambda *a: {**orig_backward(*a), "ds": orig_backward(*a)["ds"] + 0.01}),
    }
    for name, apply in mutations.items():
        with monkeypatch.context() as m:
            monkeypatch = m
            apply()
            assert _sdpa_max_err() > 1e-4, name
