"""evo_attn_bwd_noalloc: the backward without a workspace argument, for callers
that cannot allocate device memory (its scratch is a static device array).

Its outputs must match those of evo_attn_bwd, the entry point it is a variant
of, on calls in a row, each with a smaller problem than the one before (the
static array keeps the previous call's contents).  The backward fits its plan
to the workspace it is given, so evo_attn_bwd gets a workspace of exactly the
static array's size: both entry points then run the same kernels with the same
plan, and the match is exact.  One of the problems has rows longer than one
key tile and more partials than fit, so it runs in chunks.
"""
import pytest
import torch

from evoformer_biased_attention_amd import _lib
from evoformer_biased_attention_amd import inputs as I
from evoformer_biased_attention_amd.attention import attn_fwd
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

DT = {"fp16": _lib.EVO_F16, "bf16": _lib.EVO_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _backward_both_ways(cfg):
    bits = I.make_inputs(cfg)
    x = {n: to_device(bits[n], cfg.dtype) for n in ("q", "k", "v", "mask_bias", "pair_bias", "dout")}
    m, p = x["mask_bias"], x["pair_bias"]
    out, lse = attn_fwd(x["q"], x["k"], x["v"], m, p)
    stream = torch.cuda.current_stream().cuda_stream

    def outputs():
        o = {n: torch.full_like(x["q"], 7.0) for n in ("dq", "dk", "dv")}
        o["dmask"] = None if m is None else torch.full_like(m, 7.0)
        o["dpair"] = None if p is None else torch.full_like(p, 7.0)
        return o

    ref, got = outputs(), outputs()
    nws = _lib.EVO_NOALLOC_SCRATCH_BYTES
    least = _lib.evo_attn_bwd_workspace_bytes_within(cfg.shape, DT[cfg.dtype], m is not None, p is not None, 0)
    assert least <= nws
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    common = (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), _ptr(m), _ptr(p), out.data_ptr(),
              lse.data_ptr(), x["dout"].data_ptr())
    st = _lib.evo_attn_bwd(*common, ref["dq"].data_ptr(), ref["dk"].data_ptr(), ref["dv"].data_ptr(),
                           _ptr(ref["dmask"]), _ptr(ref["dpair"]), ws.data_ptr(), nws, cfg.shape, DT[cfg.dtype],
                           stream)
    assert st == 0, _lib.evo_status_string(st)
    st = _lib.evo_attn_bwd_noalloc(*common, got["dq"].data_ptr(), got["dk"].data_ptr(), got["dv"].data_ptr(),
                                   _ptr(got["dmask"]), _ptr(got["dpair"]), cfg.shape, None, DT[cfg.dtype], stream)
    assert st == 0, _lib.evo_status_string(st)
    torch.cuda.synchronize()
    for n in ref:
        if ref[n] is None:
            continue
        diff = (got[n].float() - ref[n].float()).abs().max().item()
        print(f"  {cfg.name} {n}: max |noalloc - workspace| = {diff:.3e}", flush=True)
        assert torch.equal(got[n], ref[n]), n


def test_noalloc_backward_matches_workspace_backward():
    big = I.CONFIGS["msa_row"]                                          # (1,256,256,4,32) fp16
    long_rows = I.custom("noalloc_long_rows", 1, 48, 640, 2, 64, "bf16", 0.05, 1.0, 72)
    small = I.custom("noalloc_small", 2, 5, 100, 3, 16, "bf16", 0.2, 1.0, 71)
    B, N, L, H, D = long_rows.shape
    # its dQ partials alone (5 key tiles of 128) exceed the static array: the plan goes in chunks
    assert 5 * B * N * L * H * D * 4 > _lib.EVO_NOALLOC_SCRATCH_BYTES
    for cfg in (big, long_rows, small):
        print(f"case noalloc {cfg.name} shape={cfg.shape} dtype={cfg.dtype}", flush=True)
        _backward_both_ways(cfg)
