"""Strided [B,N,L,H,D] layouts through the C ABI (GPU).

Guide §3.6 names triangle attention around the ending node beside the
starting-node form: the same operation on the pair representation transposed
over its two residue axes.  With strides the library takes that transposed
view as it is.  Every output of a strided call is compared with the fp64 oracle evaluated on
the logical tensors, and, since the arithmetic does not depend on where the
rows sit, also with the dense layout's result bit for bit:

* views transposed over N and L (the ending-node case) and permuted so that
  B is innermost, through the Python layer, forward and backward;
* rows padded past H * D through the C ABI directly: the padding of every
  output is left untouched.
"""
import numpy as np
import pytest
import torch

from evoformer_biased_attention_amd import _lib
from evoformer_biased_attention_amd import inputs as I
from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd, workspace_f32_views
from tests.helpers import compare_with_oracle, to_device

pytestmark = pytest.mark.gpu

DT = {"fp16": _lib.EVO_F16, "bf16": _lib.EVO_BF16}

CASES = [
    I.custom("str_l100_d32", 1, 6, 100, 3, 32, "fp16", 0.2, 1.0, 61),    # one tile
    I.custom("str_l77_d8_bf16", 2, 3, 77, 2, 8, "bf16", 0.2, 1.0, 62),
    I.custom("str_l300_bf16", 1, 3, 300, 2, 32, "bf16", 0.2, 1.0, 63),   # rows longer than a key tile
    I.custom("str_l200_d64", 1, 2, 200, 2, 64, "fp16", 0.2, 1.0, 64),
    I.custom("str_l96_nomask", 1, 5, 96, 2, 16, "fp16", None, 1.0, 65),
]


def _dense_inputs(cfg):
    bits = I.make_inputs(cfg)
    return {n: to_device(bits[n], cfg.dtype) for n in ("q", "k", "v", "mask_bias", "pair_bias", "dout")}


def _relayout(t, perm):
    """The same logical [B,N,L,H,D] values stored with dims B, N, L in the
    memory order `perm` (outermost first), returned as a view."""
    inv = [perm.index(d) for d in range(3)] + [3, 4]
    store = t.permute(*perm, 3, 4).contiguous()
    return store.permute(*inv)


def _run(x, q, k, v, dout, with_ws=False):
    out, lse = attn_fwd(q, k, v, x["mask_bias"], x["pair_bias"])
    g = attn_bwd(q, k, v, x["mask_bias"], x["pair_bias"], out, lse, dout)
    torch.cuda.synchronize()
    res = {"out": out, "lse": lse, "dq": g["dq"], "dk": g["dk"], "dv": g["dv"], "dmask": g["dmask"],
           "dpair": g["dpair"]}
    if with_ws:
        delta, dm32, dp32 = workspace_f32_views(g["workspace"], q.shape, q.dtype, x["mask_bias"] is not None,
                                                x["pair_bias"] is not None)
        res.update({"delta": delta.clone(), "dmask32": None if dm32 is None else dm32.clone(),
                    "dpair32": None if dp32 is None else dp32.clone()})
    return res


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_ending_node_views_against_oracle(cfg):
    """Triangle attention around the ending node: Q, K, V, dO handed over as
    views transposed over N and L (no copy) and every output, in the view's
    layout, compared with the oracle on the logical values."""
    print(f"case ending-node view vs oracle {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    bits = I.make_inputs(cfg)
    x = {n: to_device(bits[n], cfg.dtype) for n in ("q", "k", "v", "mask_bias", "pair_bias", "dout")}
    q, k, v, do = (_relayout(x[n], [0, 2, 1]) for n in ("q", "k", "v", "dout"))
    res = _run(x, q, k, v, do, with_ws=True)
    for n in ("out", "dq", "dk", "dv"):
        assert res[n].stride() == q.stride(), n
    compare_with_oracle(cfg, bits, res)


@pytest.mark.parametrize("perm", [(0, 2, 1), (2, 1, 0)], ids=["transposed_NL", "B_innermost"])
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_views_match_dense_layout(cfg, perm):
    print(f"case strided view {cfg.name} perm={perm} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    x = _dense_inputs(cfg)
    ref = _run(x, x["q"], x["k"], x["v"], x["dout"])
    q, k, v, do = (_relayout(x[n], list(perm)) for n in ("q", "k", "v", "dout"))
    assert not q.is_contiguous() or cfg.shape[0] * cfg.shape[1] == 1
    got = _run(x, q, k, v, do)
    # the outputs keep the inputs' layout (no copy was made)
    for n in ("out", "dq", "dk", "dv"):
        assert got[n].stride() == q.stride(), n
    for n, t in ref.items():
        if t is None:
            assert got[n] is None
            continue
        assert torch.equal(got[n], t), f"{n} differs from the dense layout"


@pytest.mark.parametrize("cfg", [CASES[0], CASES[2], CASES[3]], ids=[c.name for c in (CASES[0], CASES[2], CASES[3])])
def test_padded_rows_through_the_c_abi(cfg):
    print(f"case padded rows {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    B, N, L, H, D = cfg.shape
    x = _dense_inputs(cfg)
    ref = _run(x, x["q"], x["k"], x["v"], x["dout"])
    pad = 24  # elements after each row of H * D
    sL = H * D + pad
    strides = (N * L * sL, L * sL, sL)
    full = (B, N, L, sL)
    tdt = x["q"].dtype

    def padded(src=None, fill=0.0):
        buf = torch.full(full, fill, dtype=tdt, device="cuda")
        view = buf[..., :H * D].unflatten(-1, (H, D))
        if src is not None:
            view.copy_(src)
        return buf, view

    ins = {n: padded(x[n]) for n in ("q", "k", "v", "dout")}
    outs = {n: padded(fill=7.0) for n in ("out", "dq", "dk", "dv")}
    lse = torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    m, p = x["mask_bias"], x["pair_bias"]
    ptr = lambda t: None if t is None else t.data_ptr()
    assert _lib.evo_attn_fwd_strided(ins["q"][1].data_ptr(), ins["k"][1].data_ptr(), ins["v"][1].data_ptr(), ptr(m),
                                     ptr(p), outs["out"][1].data_ptr(), lse.data_ptr(), cfg.shape, strides,
                                     DT[cfg.dtype], stream) == 0
    dm = torch.empty_like(m) if m is not None else None
    dp = torch.empty_like(p) if p is not None else None
    nws = _lib.evo_attn_bwd_workspace_bytes(cfg.shape, DT[cfg.dtype], m is not None, p is not None)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    assert _lib.evo_attn_bwd_strided(ins["q"][1].data_ptr(), ins["k"][1].data_ptr(), ins["v"][1].data_ptr(), ptr(m),
                                     ptr(p), outs["out"][1].data_ptr(), lse.data_ptr(), ins["dout"][1].data_ptr(),
                                     outs["dq"][1].data_ptr(), outs["dk"][1].data_ptr(), outs["dv"][1].data_ptr(),
                                     ptr(dm), ptr(dp), ws.data_ptr(), ws.numel(), cfg.shape, strides,
                                     DT[cfg.dtype], stream) == 0
    torch.cuda.synchronize()
    for n in ("out", "dq", "dk", "dv"):
        buf, view = outs[n]
        assert torch.equal(view, ref[n]), f"{n} differs from the dense layout"
        assert bool((buf[..., H * D:] == 7.0).all()), f"padding of {n} was written"
    # the same outputs against the oracle on the logical values
    delta, dm32, dp32 = workspace_f32_views(ws, cfg.shape, tdt, m is not None, p is not None)
    res = {"out": outs["out"][1], "lse": lse, "dq": outs["dq"][1], "dk": outs["dk"][1], "dv": outs["dv"][1],
           "dmask": dm, "dpair": dp, "delta": delta, "dmask32": dm32, "dpair32": dp32}
    compare_with_oracle(cfg, I.make_inputs(cfg), res)
    assert torch.equal(lse, ref["lse"])
    if m is not None:
        assert torch.equal(dm, ref["dmask"])
    if p is not None:
        assert torch.equal(dp, ref["dpair"])
