"""fp64 CPU oracle for Evoformer biased attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP path.

What it computes is the plain definition the DeepSpeed4Science guide gives
(page "DeepSpeed4Science 技术指南", §3.5: the reference attention multiplies
QK^T by the scale factor, adds the bias, applies softmax and multiplies by V;
§3.7: the forward keeps the output and an fp32 log-sum-exp per query row, the
backward derives delta and then the gradients of Q, K, V and of both biases,
the bias gradients accumulated in fp32).  The fused kernel reaches this result
up to the order of rounding, so the oracle is that definition written out in
float64 with the full score matrix of one (b, n) slice materialised:

    S[h,i,j] = scale * sum_d q[i,h,d] k[j,h,d] + mask[j] + pair[h,i,j]
    P        = softmax_j(S),  lse[h,i] = log sum_j exp S[h,i,j]
    O[i,h,:] = sum_j P[h,i,j] v[j,h,:]

and the backward by the chain rule:

    dP = dO V^T,  dV = P^T dO,  delta_i = sum_j P_ij dP_ij,
    dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,
    dmask[b,n,j] = sum_h sum_i dS,   dpair[b,h,i,j] = sum_n dS.

Readings of points the guide leaves open (each listed in the design notes):
scale = 1/sqrt(D) with the true head dim; the biases are added after the
scale and are not scaled; the mask is an additive bias on keys only; lse is a
natural logarithm over the full biased, scaled row; a query row whose scores
are all -inf gives O = 0, lse = -inf and zero gradients.

Inputs are float64 arrays holding the exact dtype-rounded values:
q, k, v, dout [B,N,L,H,D]; mask_bias [B,N,1,1,L] or None;
pair_bias [B,1,H,L,L] or None.

Pins (tests/test_oracle.py): rows of P sum to 1; Q = 0 closed form; masked
keys contribute exactly zero; central finite differences of every input;
torch's own scaled-dot-product attention in float64 on the CPU (forward and
autograd) for the broadcast biases; textbook attention for N = H = 1 without
biases; gradient identities and invariances.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "attention_fwd",
    "attention_bwd",
    "dpair_rows",
    "slice_forward",
    "slice_backward",
]


def _scale(D: int) -> float:
    return 1.0 / np.sqrt(float(D))


def _slice_scores(qs, ks, b1, b2, scale):
    """S[h,i,j] for one (b, n) slice; qs, ks: [L,H,D]; b1: [L]|None; b2: [H,L,L]|None."""
    qh = np.ascontiguousarray(qs.transpose(1, 0, 2))  # [H, L, D]
    kh = np.ascontiguousarray(ks.transpose(1, 0, 2))
    s = scale * np.matmul(qh, kh.transpose(0, 2, 1))
    if b1 is not None:
        s = s + b1[None, None, :]
    if b2 is not None:
        s = s + b2
    return s


def _softmax_rows(s):
    """Row softmax and natural-log lse, with the all -inf row convention."""
    m = s.max(axis=-1, keepdims=True)
    dead = np.isneginf(m)
    m0 = np.where(dead, 0.0, m)
    with np.errstate(invalid="ignore"):
        e = np.exp(s - m0)
    e = np.where(dead, 0.0, e)
    l = e.sum(axis=-1, keepdims=True)
    p = e / np.where(dead, 1.0, l)
    with np.errstate(divide="ignore"):
        lse = np.where(dead, -np.inf, m0 + np.log(np.where(dead, 1.0, l)))
    return p, lse[..., 0]


def slice_forward(qs, ks, vs, b1, b2) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Forward of one (b, n) slice.  Returns (O [L,H,D], lse [H,L], P [H,L,L])."""
    scale = _scale(qs.shape[-1])
    s = _slice_scores(qs, ks, b1, b2, scale)
    p, lse = _softmax_rows(s)
    vh = vs.transpose(1, 0, 2)
    o = np.matmul(p, vh).transpose(1, 0, 2)
    return o, lse, p


def slice_backward(qs, ks, vs, b1, b2, dos) -> Dict[str, np.ndarray]:
    """Backward of one (b, n) slice by the chain rule.

    Returns dq, dk, dv [L,H,D]; dmask [L]; ds [H,L,L] (this slice's share of
    dpair); delta [H,L].
    """
    scale = _scale(qs.shape[-1])
    _, _, p = slice_forward(qs, ks, vs, b1, b2)
    qh = qs.transpose(1, 0, 2)
    kh = ks.transpose(1, 0, 2)
    vh = vs.transpose(1, 0, 2)
    doh = dos.transpose(1, 0, 2)
    dp = np.matmul(doh, vh.transpose(0, 2, 1))  # [H, Lq, Lk]
    dv = np.matmul(p.transpose(0, 2, 1), doh)  # [H, Lk, D]
    delta = (p * dp).sum(axis=-1)  # [H, Lq]
    ds = p * (dp - delta[..., None])
    dq = scale * np.matmul(ds, kh)
    dk = scale * np.matmul(ds.transpose(0, 2, 1), qh)
    return {
        "dq": dq.transpose(1, 0, 2),
        "dk": dk.transpose(1, 0, 2),
        "dv": dv.transpose(1, 0, 2),
        "dmask": ds.sum(axis=(0, 1)),
        "ds": ds,
        "delta": delta,
    }


def _bias_slices(mask_bias, pair_bias, b, n):
    b1 = None if mask_bias is None else mask_bias[b, n, 0, 0, :]
    b2 = None if pair_bias is None else pair_bias[b, 0]
    return b1, b2


def _slices(B: int, N: int, ns: Optional[Iterable[int]]):
    nlist = list(range(N)) if ns is None else [int(x) for x in ns]
    return [(b, n) for b in range(B) for n in nlist], nlist


def attention_fwd(q, k, v, mask_bias=None, pair_bias=None, ns: Optional[Sequence[int]] = None):
    """Forward over all slices, or only over dim-1 indices ``ns``.

    Returns O [B,len(ns),L,H,D] and lse [B,len(ns),H,L] (float64).
    """
    B, N, L, H, D = q.shape
    pairs, nlist = _slices(B, N, ns)
    out = np.zeros((B, len(nlist), L, H, D))
    lse = np.zeros((B, len(nlist), H, L))
    for b, n in pairs:
        b1, b2 = _bias_slices(mask_bias, pair_bias, b, n)
        o, l, _ = slice_forward(q[b, n], k[b, n], v[b, n], b1, b2)
        t = nlist.index(n)
        out[b, t] = o
        lse[b, t] = l
    return out, lse


def attention_bwd(q, k, v, mask_bias, pair_bias, dout, ns: Optional[Sequence[int]] = None):
    """Gradients over all slices, or only over dim-1 indices ``ns``.

    dq, dk, dv [B,len(ns),L,H,D]; dmask [B,len(ns),1,1,L] (None without a
    mask); delta [B,len(ns),H,L].  dpair [B,1,H,L,L] sums over n, so it is
    returned only when every slice is computed (ns is None); otherwise use
    :func:`dpair_rows`.
    """
    B, N, L, H, D = q.shape
    pairs, nlist = _slices(B, N, ns)
    dq = np.zeros((B, len(nlist), L, H, D))
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    dmask = np.zeros((B, len(nlist), 1, 1, L))
    delta = np.zeros((B, len(nlist), H, L))
    dpair = np.zeros((B, 1, H, L, L)) if (ns is None and pair_bias is not None) else None
    for b, n in pairs:
        b1, b2 = _bias_slices(mask_bias, pair_bias, b, n)
        g = slice_backward(q[b, n], k[b, n], v[b, n], b1, b2, dout[b, n])
        t = nlist.index(n)
        dq[b, t], dk[b, t], dv[b, t] = g["dq"], g["dk"], g["dv"]
        dmask[b, t, 0, 0] = g["dmask"]
        delta[b, t] = g["delta"]
        if dpair is not None:
            dpair[b, 0] += g["ds"]
    return {
        "dq": dq,
        "dk": dk,
        "dv": dv,
        "dmask": dmask if mask_bias is not None else None,
        "dpair": dpair,
        "delta": delta,
    }


def dpair_rows(q, k, v, mask_bias, pair_bias, dout, rows: Sequence[Tuple[int, int, int]]):
    """dpair[b,h,i,:] for selected (b, h, i), summing dS over every n.

    Same definition as :func:`attention_bwd`, evaluated one query row at a
    time: for each n, the row S[h,i,:], its softmax P, dP[h,i,:] = dO_i V^T,
    delta_i = sum_j P dP and dS = P (dP - delta_i).
    Returns an array [len(rows), L].
    """
    B, N, L, H, D = q.shape
    scale = _scale(D)
    res = np.zeros((len(rows), L))
    for r, (b, h, i) in enumerate(rows):
        # all n at once: S[n, j] for the fixed query row i of head h
        s = scale * np.einsum("njd,nd->nj", k[b, :, :, h, :], q[b, :, i, h, :])
        if mask_bias is not None:
            s = s + mask_bias[b, :, 0, 0, :]
        if pair_bias is not None:
            s = s + pair_bias[b, 0, h, i, :][None, :]
        p, _ = _softmax_rows(s)
        dp = np.einsum("njd,nd->nj", v[b, :, :, h, :], dout[b, :, i, h, :])
        delta = (p * dp).sum(axis=-1, keepdims=True)
        res[r] = (p * (dp - delta)).sum(axis=0)
    return res
