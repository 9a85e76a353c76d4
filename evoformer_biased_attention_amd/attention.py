"""PyTorch-facing API: DS4Sci_EvoformerAttention-style call over the C ABI.

torch provides device memory and the current stream; every operation runs in
the library's HIP kernels (see _lib.py).  Interface per the DeepSpeed4Science
guide, §3.6-§3.7: ``evoformer_attention(Q, K, V, biases)`` with ``biases`` a
list of at most two tensors, [B,N,1,1,L] (mask) and [B,1,H,L,L] (pair); a
missing slot is treated as absent; inputs must be fp16 or bf16 on the current
GPU; gradients flow to Q, K, V and both biases through autograd.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import _lib

_DT = {torch.float16: _lib.EVO_F16, torch.bfloat16: _lib.EVO_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_inputs(q, k, v, mask, pair):
    if q.dtype not in _DT:
        raise TypeError(f"inputs must be float16 or bfloat16, got {q.dtype}")
    for name, t in (("k", k), ("v", v), ("mask_bias", mask), ("pair_bias", pair)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    if q.dim() != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"Q, K, V must share one [B,N,L,H,D] shape, got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    B, N, L, H, D = q.shape
    if mask is not None and tuple(mask.shape) != (B, N, 1, 1, L):
        raise ValueError(f"bias 1 must be [B,N,1,1,L] = {(B, N, 1, 1, L)}, got {tuple(mask.shape)}")
    if pair is not None and tuple(pair.shape) != (B, 1, H, L, L):
        raise ValueError(f"bias 2 must be [B,1,H,L,L] = {(B, 1, H, L, L)}, got {tuple(pair.shape)}")


def _layout(ts) -> Optional[Tuple[int, int, int]]:
    """The (sB, sN, sL) element strides that the [B,N,L,H,D] tensors ``ts`` share,
    when the library can take them as they are: the same strides for all, the
    H heads of D elements of each row dense, and the tensor dense as a whole
    (a permutation of the B, N, L dims, such as a view transposed over N and L).
    None otherwise (the caller then makes the tensors contiguous)."""
    t0 = ts[0]
    B, N, L, H, D = t0.shape
    if all(t.is_contiguous() for t in ts):
        return _dense_strides(t0.shape)
    st = t0.stride()
    if any(t.stride() != st for t in ts[1:]):
        return None
    if st[4] != 1 or (H > 1 and st[3] != D):
        return None
    # dense as a whole: the dims of extent > 1, in increasing stride order, each
    # start where the ones below end (the first right after one row of H * D)
    span = H * D
    for x, e in sorted((x, e) for x, e in zip(st[:3], (B, N, L)) if e > 1):
        if x != span:
            return None
        span = x * e
    # a dim of extent 1 may carry any stride: give it one the library accepts
    return tuple(x if e > 1 else 8 for x, e in zip(st[:3], (B, N, L)))


def _aligned(t: Optional[torch.Tensor], contiguous: bool = False) -> Optional[torch.Tensor]:
    """``t`` itself when the library can take it, else a fresh copy: the C ABI needs
    16-byte aligned pointers, which a valid view at an odd element offset (a
    slice of a larger tensor) does not have.  ``contiguous`` also makes the
    result dense row-major (the bias and lse layouts the library assumes)."""
    if t is None:
        return None
    if contiguous:
        t = t.contiguous()
    if t.data_ptr() % 16 != 0:
        t = t.clone(memory_format=torch.contiguous_format if contiguous else torch.preserve_format)
    return t


def _dense_strides(shape) -> Tuple[int, int, int]:
    B, N, L, H, D = shape
    return (N * L * H * D, L * H * D, H * D)


def _empty_problem(q: torch.Tensor) -> bool:
    """A problem with no score at all (B, N, L or H zero, a supported D): there
    is nothing to compute, and the library, whose shapes are at least 1, is
    not called."""
    B, N, L, H, D = q.shape
    return q.numel() == 0 and D in (8, 16, 32, 64)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask_bias: Optional[torch.Tensor] = None,
             pair_bias: Optional[torch.Tensor] = None, need_lse: bool = True
             ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward: returns (out [B,N,L,H,D] dtype, lse [B,N,H,L] float32).

    With ``need_lse=False`` (inference: no backward follows) the lse is neither
    allocated nor written and None is returned in its place; out is identical.
    """
    _check_inputs(q, k, v, mask_bias, pair_bias)
    if _empty_problem(q):
        B, N, L, H, D = q.shape
        out = torch.empty_like(q)
        return out, (torch.empty((B, N, H, L), dtype=torch.float32, device=q.device) if need_lse else None)
    lay = _layout((q, k, v))
    if lay is None:
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        lay = _dense_strides(q.shape)
    q, k, v = _aligned(q), _aligned(k), _aligned(v)
    mask_bias = _aligned(mask_bias, contiguous=True)
    pair_bias = _aligned(pair_bias, contiguous=True)
    B, N, L, H, D = q.shape
    out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, N, H, L), dtype=torch.float32, device=q.device) if need_lse else None
    _lib.check(_lib.evo_attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(mask_bias),
                                         _ptr(pair_bias), out.data_ptr(), _ptr(lse), q.shape, lay, _DT[q.dtype],
                                         _stream()))
    return out, lse


def attn_bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, want_dmask: bool = True, want_dpair: bool = True,
             workspace: Optional[torch.Tensor] = None,
             partial_budget: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Backward: returns dict dq, dk, dv, dmask (or None), dpair (or None), workspace.

    The library fits its plan to the workspace: a given `workspace` is used as
    it is (it must hold at least the least workspace the backward accepts);
    otherwise one is allocated, of the default size or of the size for
    `partial_budget` bytes of fp32 partials (long rows then go in chunks).
    A problem with no score returns empty gradients, and bias gradients that
    sum over an empty dimension (dpair with N = 0, dmask with H = 0) are zero."""
    _check_inputs(q, k, v, mask_bias, pair_bias)
    if _empty_problem(q):
        return {"dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q),
                "dmask": torch.zeros_like(mask_bias) if (mask_bias is not None and want_dmask) else None,
                "dpair": torch.zeros_like(pair_bias) if (pair_bias is not None and want_dpair) else None,
                "workspace": workspace if workspace is not None else torch.empty(0, dtype=torch.uint8,
                                                                                  device=q.device)}
    lay = _layout((q, k, v, out))
    if lay is None:
        q, k, v, out = (t.contiguous() for t in (q, k, v, out))
        lay = _dense_strides(q.shape)
    q, k, v, out = _aligned(q), _aligned(k), _aligned(v), _aligned(out)
    if dout.stride() != q.stride() or dout.data_ptr() % 16 != 0:
        dout = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device).copy_(dout)
    lse = _aligned(lse, contiguous=True)
    mask_bias = _aligned(mask_bias, contiguous=True)
    pair_bias = _aligned(pair_bias, contiguous=True)
    B, N, L, H, D = q.shape
    dt = _DT[q.dtype]
    dq, dk, dv = (torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) for _ in range(3))
    dmask = torch.empty_like(mask_bias) if (mask_bias is not None and want_dmask) else None
    dpair = torch.empty_like(pair_bias) if (pair_bias is not None and want_dpair) else None
    hm, hp = mask_bias is not None, pair_bias is not None
    if workspace is None:
        if partial_budget is None:
            nbytes = _lib.evo_attn_bwd_workspace_bytes(q.shape, dt, hm, hp)
        else:
            nbytes = _lib.evo_attn_bwd_workspace_bytes_within(q.shape, dt, hm, hp, partial_budget)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() < _lib.evo_attn_bwd_workspace_bytes_within(q.shape, dt, hm, hp, 0):
        raise ValueError("workspace smaller than the least the backward accepts")
    _lib.check(_lib.evo_attn_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), _ptr(mask_bias),
                                         _ptr(pair_bias), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _ptr(dmask), _ptr(dpair),
                                         workspace.data_ptr(), workspace.numel(), q.shape, lay, dt, _stream()))
    return {"dq": dq, "dk": dk, "dv": dv, "dmask": dmask, "dpair": dpair, "workspace": workspace}


def workspace_f32_views(workspace: torch.Tensor, shape, dtype: torch.dtype, has_mask: bool, has_pair: bool):
    """fp32 views of delta, dmask and dpair accumulators inside a backward workspace."""
    B, N, L, H, D = shape
    od, om, op = _lib.evo_attn_bwd_workspace_offsets(shape, _DT[dtype], has_mask, has_pair)

    def view(off, n, shp):
        if off is None:
            return None
        return workspace[off:off + 4 * n].view(torch.float32).view(*shp)

    return (view(od, B * N * H * L, (B, N, H, L)),
            view(om, B * N * L, (B, N, 1, 1, L)),
            view(op, B * H * L * L, (B, 1, H, L, L)))


class EvoformerFusedAttention(torch.autograd.Function):
    """Autograd wrapper: forward saves Q, K, V, biases, O and lse; backward recomputes."""

    @staticmethod
    def forward(ctx, q, k, v, mask_bias, pair_bias):
        out, lse = attn_fwd(q, k, v, mask_bias, pair_bias)
        ctx.save_for_backward(q, k, v, mask_bias, pair_bias, out, lse)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, mask_bias, pair_bias, out, lse = ctx.saved_tensors
        want_m = mask_bias is not None and ctx.needs_input_grad[3]
        want_p = pair_bias is not None and ctx.needs_input_grad[4]
        g = attn_bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, want_m, want_p)
        return g["dq"], g["dk"], g["dv"], g["dmask"], g["dpair"]


def evoformer_attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                        biases: Sequence[Optional[torch.Tensor]] = ()) -> torch.Tensor:
    """softmax(Q K^T / sqrt(D) + biases) V over [B, N, L, H, D] tensors.

    ``biases`` holds at most two tensors: [B,N,1,1,L] and [B,1,H,L,L]; a
    missing slot is treated as absent (guide §3.7).
    """
    bl: List[Optional[torch.Tensor]] = list(biases)
    if len(bl) > 2:
        raise ValueError("at most two biases: [B,N,1,1,L] and [B,1,H,L,L]")
    while len(bl) < 2:
        bl.append(None)
    if not (torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in (Q, K, V, *bl))):
        # no gradient can flow: the inference forward, which keeps no lse
        return attn_fwd(Q, K, V, bl[0], bl[1], need_lse=False)[0]
    return EvoformerFusedAttention.apply(Q, K, V, bl[0], bl[1])


DS4Sci_EvoformerAttention = evoformer_attention
