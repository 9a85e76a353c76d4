"""Properties of the HIP path that hold exactly, at any size, plus the C ABI's
error behaviour on a real device.

* masked keys: changing K and V at keys whose mask is -1e9 changes no output
  bit; dK, dV and dmask are exactly zero there (P is exactly zero at those keys);
* determinism: two runs give the same bits (every path, rows longer than one
  key tile included: every reduction runs in a fixed order, no atomics), and
  repeated backward calls at sizes that fill the device do too;
* inference forward (no lse kept): the same output bits as the forward that
  keeps the lse, through the C ABI and through the no-grad Python call;
* coverage: outputs pre-filled with NaN come back finite (every element written);
* guard bands: bytes just before and after every output and the workspace are
  left untouched;
* streams: a run on a side stream gives the same bits as on the current stream;
* argument errors (host pointer, misaligned pointer, short workspace, a bias
  gradient without its bias, an output aliasing an input) return their status
  and leave every output untouched;
* empty problems (B, N, L or H zero) through the Python layer: outputs of the
  right empty shapes, and the bias gradient that sums over an empty dimension
  (dpair with N = 0, dmask with H = 0) is exactly zero.
"""
import numpy as np
import pytest
import torch

from evoformer_biased_attention_amd import _lib
from evoformer_biased_attention_amd import inputs as I
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

DT = {"fp16": _lib.EVO_F16, "bf16": _lib.EVO_BF16}
GUARD = 256  # bytes of guard band on each side


def _inputs(cfg):
    bits = I.make_inputs(cfg)
    return bits, {n: to_device(bits[n], cfg.dtype) for n in ("q", "k", "v", "mask_bias", "pair_bias", "dout")}


def _guarded(shape, dtype, fill):
    """A tensor view with GUARD bytes of `fill` bytes on each side inside one allocation."""
    esize = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape))
    raw = torch.full((2 * GUARD + n * esize,), fill, dtype=torch.uint8, device="cuda")
    body = raw[GUARD:GUARD + n * esize].view(dtype).view(*shape)
    return raw, body


def _ptr(t):
    return None if t is None else t.data_ptr()


def _run(cfg, x, fill=0xFF, stream=None, ws_extra=0):
    """fwd + bwd through the C ABI into guarded buffers pre-filled with `fill` bytes
    (0xFF makes fp16/bf16/fp32 NaN)."""
    B, N, L, H, D = cfg.shape
    tdt = x["q"].dtype
    st = torch.cuda.current_stream() if stream is None else stream
    has_m, has_p = x["mask_bias"] is not None, x["pair_bias"] is not None
    bufs = {}
    for name, shp, dt in (("out", cfg.shape, tdt), ("lse", (B, N, H, L), torch.float32), ("dq", cfg.shape, tdt),
                          ("dk", cfg.shape, tdt), ("dv", cfg.shape, tdt)):
        bufs[name] = _guarded(shp, dt, fill)
    if has_m:
        bufs["dmask"] = _guarded((B, N, 1, 1, L), tdt, fill)
    if has_p:
        bufs["dpair"] = _guarded((B, 1, H, L, L), tdt, fill)
    nws = _lib.evo_attn_bwd_workspace_bytes(cfg.shape, DT[cfg.dtype], has_m, has_p)
    bufs["ws"] = _guarded((nws + ws_extra,), torch.uint8, fill)
    body = {k: v[1] for k, v in bufs.items()}
    with torch.cuda.stream(st):
        _lib.check(_lib.evo_attn_fwd(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), _ptr(x["mask_bias"]),
                                     _ptr(x["pair_bias"]), body["out"].data_ptr(), body["lse"].data_ptr(), cfg.shape,
                                     DT[cfg.dtype], st.cuda_stream))
        _lib.check(_lib.evo_attn_bwd(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), _ptr(x["mask_bias"]),
                                     _ptr(x["pair_bias"]), body["out"].data_ptr(), body["lse"].data_ptr(),
                                     x["dout"].data_ptr(), body["dq"].data_ptr(), body["dk"].data_ptr(),
                                     body["dv"].data_ptr(), _ptr(body.get("dmask")), _ptr(body.get("dpair")),
                                     body["ws"].data_ptr(), nws, cfg.shape, DT[cfg.dtype], st.cuda_stream))
    torch.cuda.synchronize()
    return bufs


def _outputs(bufs):
    return {k: v[1] for k, v in bufs.items() if k != "ws"}


def _assert_guards(bufs, fill):
    for name, (raw, body) in bufs.items():
        nb = body.numel() * body.element_size()
        head, tail = raw[:GUARD], raw[GUARD + nb:]
        assert bool((head == fill).all()) and bool((tail == fill).all()), f"guard band of {name} was written"


CASES = [
    I.custom("inv_l77_bf16", 2, 3, 77, 2, 16, "bf16", 0.25, 1.0, 31),
    I.custom("inv_l100_d32", 1, 5, 100, 3, 32, "fp16", 0.25, 1.0, 32),
    I.custom("inv_l200_d64", 1, 3, 200, 2, 64, "fp16", 0.25, 1.0, 33),
    I.custom("inv_l256_d8_bf16", 1, 4, 256, 4, 8, "bf16", 0.25, 1.0, 34),
    I.custom("inv_l300_bf16", 1, 2, 300, 2, 32, "bf16", 0.25, 1.0, 35),
    I.custom("inv_l520_d16", 1, 2, 520, 1, 16, "fp16", 0.25, 1.0, 36),
    I.custom("inv_l600_nopair_bf16", 1, 3, 600, 2, 32, "bf16", 0.25, None, 37),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_every_output_written_guards_intact_deterministic(cfg):
    print(f"case coverage/guards {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    _, x = _inputs(cfg)
    a = _run(cfg, x, fill=0xFF)
    _assert_guards(a, 0xFF)
    for name, t in _outputs(a).items():
        assert bool(torch.isfinite(t.float()).all()), f"{name} has unwritten (NaN) elements"
    b = _run(cfg, x, fill=0x00)
    _assert_guards(b, 0x00)
    for name in _outputs(a):
        assert torch.equal(_outputs(a)[name], _outputs(b)[name]), f"{name} differs between two runs"


REPEAT = [
    I.custom("rep_l640_d32_bf16", 2, 8, 640, 2, 32, "bf16", 0.05, 1.0, 52),
    I.custom("rep_l128_d64_bf16", 1, 8, 128, 2, 64, "bf16", 0.05, 1.0, 54),
    I.custom("rep_l256_d32", 1, 16, 256, 4, 32, "fp16", 0.05, 1.0, 55),
]


@pytest.mark.parametrize("cfg", REPEAT, ids=[c.name for c in REPEAT])
def test_backward_bits_repeat(cfg):
    """Several backward calls on the same inputs give the same bits, at sizes that
    keep every CU busy (a product that reads an accumulator before it is written
    shows up here as outputs that change from call to call)."""
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd

    print(f"case repeat {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    _, x = _inputs(cfg)
    out, lse = attn_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"])
    ref = None
    for rep in range(4):
        g = attn_bwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], out, lse, x["dout"])
        torch.cuda.synchronize()
        got = {k: g[k].clone() for k in ("dq", "dk", "dv", "dmask", "dpair")}
        if ref is None:
            ref = got
            continue
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"{k} differs on call {rep}"


@pytest.mark.parametrize("cfg", CASES[:4] + [CASES[5]], ids=[c.name for c in CASES[:4] + [CASES[5]]])
def test_masked_keys_are_inert(cfg):
    print(f"case masked keys {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    bits, x = _inputs(cfg)
    masked = torch.from_numpy(I.as_float64(bits, cfg.dtype)["mask_bias"][:, :, 0, 0, :] < -1e8).cuda()  # [B,N,L]
    assert bool(masked.any())
    ref = _outputs(_run(cfg, x))
    y = dict(x)
    sel = masked[:, :, :, None, None].expand_as(x["k"])
    g = torch.Generator(device="cuda").manual_seed(77)
    y["k"] = torch.where(sel, torch.randn(x["k"].shape, device="cuda", generator=g).mul(30).to(x["k"].dtype), x["k"])
    y["v"] = torch.where(sel, torch.randn(x["v"].shape, device="cuda", generator=g).mul(30).to(x["v"].dtype), x["v"])
    got = _outputs(_run(cfg, y))
    for name in ("out", "lse", "dq", "dmask", "dpair"):
        assert torch.equal(got[name], ref[name]), f"{name} changed when masked K/V changed"
    for name in ("dk", "dv"):
        z = got[name][sel]
        assert bool((z == 0).all()), f"{name} is not zero at masked keys"
        assert torch.equal(got[name][~sel], ref[name][~sel]), f"{name} changed at unmasked keys"
    dm = got["dmask"][:, :, 0, 0, :]
    assert bool((dm[masked] == 0).all()), "dmask is not zero at masked keys"


def test_side_stream_matches_current_stream():
    cfg = I.CONFIGS["msa_row"]
    print(f"case side stream msa_row shape={cfg.shape}", flush=True)
    _, x = _inputs(cfg)
    a = _outputs(_run(cfg, x))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    b = _outputs(_run(cfg, x, stream=s))
    for name in a:
        assert torch.equal(a[name], b[name]), f"{name} differs on a side stream"


def test_autograd_wrapper_equals_direct_calls():
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd, evoformer_attention

    cfg = I.custom("autograd_l64", 1, 3, 64, 2, 32, "bf16", 0.2, 1.0, 41)
    print(f"case autograd {cfg.name}", flush=True)
    _, x = _inputs(cfg)
    leaves = {n: x[n].clone().requires_grad_(True) for n in ("q", "k", "v", "mask_bias", "pair_bias")}
    out = evoformer_attention(leaves["q"], leaves["k"], leaves["v"], [leaves["mask_bias"], leaves["pair_bias"]])
    out.backward(x["dout"])
    o2, lse2 = attn_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"])
    g2 = attn_bwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], o2, lse2, x["dout"])
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o2)
    for n, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("mask_bias", "dmask"), ("pair_bias", "dpair")):
        assert torch.equal(leaves[n].grad, g2[key]), n
    # one bias only (column attention): the missing slot is absent
    out_m = evoformer_attention(x["q"], x["k"], x["v"], [x["mask_bias"]])
    o3, _ = attn_fwd(x["q"], x["k"], x["v"], x["mask_bias"], None)
    assert torch.equal(out_m, o3)


@pytest.mark.parametrize("shape", [(0, 3, 16, 2, 32), (2, 0, 16, 2, 32), (1, 3, 0, 2, 16), (1, 3, 16, 0, 8)],
                         ids=["B0", "N0", "L0", "H0"])
def test_empty_problems(shape):
    from evoformer_biased_attention_amd.attention import evoformer_attention

    print(f"case empty {shape}", flush=True)
    B, N, L, H, D = shape
    g = torch.Generator(device="cpu").manual_seed(5)
    mk = lambda *s_: torch.randn(*s_, generator=g).to("cuda", torch.float16).requires_grad_(True)
    q, k, v = mk(B, N, L, H, D), mk(B, N, L, H, D), mk(B, N, L, H, D)
    m, p = mk(B, N, 1, 1, L), mk(B, 1, H, L, L)
    out = evoformer_attention(q, k, v, [m, p])
    assert out.shape == q.shape and out.numel() == 0
    out.backward(torch.zeros_like(out))
    torch.cuda.synchronize()
    for t in (q, k, v):
        assert t.grad.shape == t.shape
    assert m.grad.shape == m.shape and p.grad.shape == p.shape
    # sums over an empty dimension are zero
    assert bool((m.grad == 0).all()) and bool((p.grad == 0).all())
    if N == 0 and B * H * L > 0:
        assert p.grad.numel() > 0
    if H == 0 and B * N * L > 0:
        assert m.grad.numel() > 0
    with torch.no_grad():
        assert evoformer_attention(q, k, v, [m, p]).shape == q.shape


def test_offset_views_are_taken():
    """Valid views at an odd element offset (slices of larger tensors) have
    pointers that are not 16-byte aligned, which the C ABI refuses; the Python
    layer hands the library aligned copies, and the results equal those of the
    aligned tensors bit for bit."""
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd, evoformer_attention

    cfg = I.custom("offset_l36", 1, 3, 36, 2, 16, "fp16", 0.2, 1.0, 42)
    print(f"case offset views {cfg.name}", flush=True)
    _, x = _inputs(cfg)

    def offset(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        view = buf[1:].view(t.shape)
        view.copy_(t)
        assert view.data_ptr() % 16 != 0
        return view

    y = {n: offset(t) for n, t in x.items()}
    o1, l1 = attn_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"])
    o2, l2 = attn_fwd(y["q"], y["k"], y["v"], y["mask_bias"], y["pair_bias"])
    g1 = attn_bwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], o1, l1, x["dout"])
    g2 = attn_bwd(y["q"], y["k"], y["v"], y["mask_bias"], y["pair_bias"], offset(o1), offset(l1), y["dout"])
    with torch.no_grad():
        o3 = evoformer_attention(y["q"], y["k"], y["v"], [y["mask_bias"], y["pair_bias"]])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)
    for key in ("dq", "dk", "dv", "dmask", "dpair"):
        assert torch.equal(g1[key], g2[key]), key


@pytest.mark.parametrize("cfg", [CASES[0], CASES[2], CASES[4], CASES[5]], ids=[c.name for c in (CASES[0], CASES[2], CASES[4], CASES[5])])
def test_inference_forward_same_output(cfg):
    from evoformer_biased_attention_amd.attention import attn_fwd, evoformer_attention

    print(f"case inference fwd {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
    _, x = _inputs(cfg)
    ref, lse = attn_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"])
    raw, body = _guarded(cfg.shape, x["q"].dtype, 0xFF)
    st = _lib.evo_attn_fwd(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), _ptr(x["mask_bias"]),
                           _ptr(x["pair_bias"]), body.data_ptr(), None, cfg.shape, DT[cfg.dtype],
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(body, ref), "out differs when no lse is kept"
    nb = body.numel() * body.element_size()
    assert bool((raw[:GUARD] == 0xFF).all()) and bool((raw[GUARD + nb:] == 0xFF).all())
    out2, none = attn_fwd(x["q"], x["k"], x["v"], x["mask_bias"], x["pair_bias"], need_lse=False)
    assert none is None and torch.equal(out2, ref)
    with torch.no_grad():
        out3 = evoformer_attention(x["q"], x["k"], x["v"], [x["mask_bias"], x["pair_bias"]])
    assert torch.equal(out3, ref)


# ---- argument errors on a real device ----

def _sentinel_outputs(cfg, x):
    B, N, L, H, D = cfg.shape
    tdt = x["q"].dtype
    o = {n: torch.full(cfg.shape, 7.0, dtype=tdt, device="cuda") for n in ("out", "dq", "dk", "dv")}
    o["lse"] = torch.full((B, N, H, L), 7.0, device="cuda")
    o["dmask"] = torch.full((B, N, 1, 1, L), 7.0, dtype=tdt, device="cuda")
    o["dpair"] = torch.full((B, 1, H, L, L), 7.0, dtype=tdt, device="cuda")
    return o


def _untouched(o):
    torch.cuda.synchronize()
    for n, t in o.items():
        assert bool((t == 7.0).all()), f"{n} was written by a failing call"


def _fwd(cfg, x, o, **over):
    a = dict(q=x["q"].data_ptr(), k=x["k"].data_ptr(), v=x["v"].data_ptr(), m=_ptr(x["mask_bias"]),
             p=_ptr(x["pair_bias"]), out=o["out"].data_ptr(), lse=o["lse"].data_ptr())
    a.update(over)
    return _lib.evo_attn_fwd(a["q"], a["k"], a["v"], a["m"], a["p"], a["out"], a["lse"], cfg.shape, DT[cfg.dtype],
                             torch.cuda.current_stream().cuda_stream)


def _bwd(cfg, x, o, ws_t, nws, **over):
    a = dict(q=x["q"].data_ptr(), k=x["k"].data_ptr(), v=x["v"].data_ptr(), m=_ptr(x["mask_bias"]),
             p=_ptr(x["pair_bias"]), out=o["out"].data_ptr(), lse=o["lse"].data_ptr(), do=x["dout"].data_ptr(),
             dq=o["dq"].data_ptr(), dk=o["dk"].data_ptr(), dv=o["dv"].data_ptr(), dm=o["dmask"].data_ptr(),
             dp=o["dpair"].data_ptr(), ws=ws_t.data_ptr(), nws=nws)
    a.update(over)
    return _lib.evo_attn_bwd(a["q"], a["k"], a["v"], a["m"], a["p"], a["out"], a["lse"], a["do"], a["dq"], a["dk"],
                             a["dv"], a["dm"], a["dp"], a["ws"], a["nws"], cfg.shape, DT[cfg.dtype],
                             torch.cuda.current_stream().cuda_stream)


def test_argument_errors_leave_outputs_untouched():
    cfg = I.custom("abi_errors", 1, 2, 40, 2, 16, "fp16", 0.1, 1.0, 51)
    print("case ABI errors on device", flush=True)
    _, x = _inputs(cfg)
    o = _sentinel_outputs(cfg, x)
    nws = _lib.evo_attn_bwd_workspace_bytes(cfg.shape, DT[cfg.dtype], True, True)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    host_q = x["q"].cpu()
    pinned_k = x["k"].cpu().pin_memory()
    mis = torch.empty(x["q"].numel() * 2 + 64, dtype=torch.uint8, device="cuda")
    mis_ptr = mis.data_ptr() + 2

    assert _fwd(cfg, x, o, q=host_q.data_ptr()) == 6          # EVO_ERR_NOT_DEVICE_MEMORY
    assert _fwd(cfg, x, o, k=pinned_k.data_ptr()) == 6
    assert _fwd(cfg, x, o, v=mis_ptr) == 5                     # EVO_ERR_ALIGNMENT
    assert _fwd(cfg, x, o, out=x["q"].data_ptr()) == 10        # EVO_ERR_ALIAS
    assert _fwd(cfg, x, o, lse=o["out"].data_ptr()) == 10
    assert _fwd(cfg, x, o, q=None) == 1                        # EVO_ERR_NULL_POINTER
    assert _bwd(cfg, x, o, ws, nws - 16) == 7                 # EVO_ERR_WORKSPACE (short)
    assert _bwd(cfg, x, o, ws, nws, ws=None) == 7
    assert _bwd(cfg, x, o, ws, nws, m=None) == 1               # dmask requested without the mask
    assert _bwd(cfg, x, o, ws, nws, p=None) == 1               # dpair requested without the pair bias
    assert _bwd(cfg, x, o, ws, nws, dq=o["dk"].data_ptr()) == 10
    assert _bwd(cfg, x, o, ws, nws, dv=x["dout"].data_ptr()) == 10
    assert _bwd(cfg, x, o, ws, nws, do=host_q.data_ptr()) == 6
    assert _bwd(cfg, x, o, ws, nws, ws=mis_ptr) == 5
    _untouched(o)
    # the error left nothing behind: a valid call right after succeeds and writes
    assert _fwd(cfg, x, o) == 0
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o["out"].float()).all()) and not bool((o["lse"] == 7.0).any())
