"""PyTorch-facing wrappers of libgdr: allocation of outputs and workspace with
the torch caching allocator on the current stream, and a thin autograd
Function.  Argument marshalling only -- every step of the computation runs
in libgdr's HIP kernels (loaded through ``_lib``; missing library = error).

The features follow FlashQLA PR #34 ("SM120/121 : Add support for fused
backward kernel", section "Current status"): fixed-length and packed
variable-length inputs, KV/VK state layouts, initial and final states,
autograd, intra-card context parallelism (``cp_segments``, which the
forward and the backward may set differently).  ``h_store`` selects the dtype
of the per-chunk state snapshots (the fp16 ``h_dtype`` of the PR's draft page
is ``h_store="f16"``).
"""
from __future__ import annotations

import os
from typing import Optional

import torch

from . import _lib

_IO = {torch.bfloat16: _lib.GDR_BF16, torch.float32: _lib.GDR_F32}
_HS = {"f32": _lib.GDR_F32, "f16": _lib.GDR_F16, "bf16": _lib.GDR_BF16}
_HS_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_LAYOUT = {"KV": _lib.GDR_LAYOUT_KV, "VK": _lib.GDR_LAYOUT_VK}


def make_problem(q: torch.Tensor, v: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                 layout: str = "KV", scale: Optional[float] = None, h_store: str = "f32",
                 cp_segments: int = 1) -> _lib.gdr_problem:
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B, T, H, DK] and v [B, T, H, DV]")
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if q.dtype not in _IO:
        raise ValueError("q, k, v must be bfloat16 or float32 (got %s)" % q.dtype)
    p = _lib.gdr_problem()
    p.batch, p.seqlen, p.heads, p.dk, p.dv, p.chunk = B, T, H, DK, DV, 64
    p.varlen = 1 if cu_seqlens is not None else 0
    p.num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    p.io_dtype = _IO[q.dtype]
    p.h_store_dtype = _HS[h_store]
    p.layout = _LAYOUT[layout]
    p.cp_segments = cp_segments
    p.scale = float(scale) if scale is not None else 0.0
    return p


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _check_tensors(q, k, v, beta, g, cu_seqlens, extra=()):
    # shapes first: the kernels take B, T and H from q and address every
    # [B, T, H, ...] tensor with them, so a shorter v (or dO) would be read
    # past its end
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B, T, H, DK] and v [B, T, H, DV]")
    if k.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q and k must match in shape and dtype; v must match their dtype")
    if v.shape[:3] != q.shape[:3]:
        raise ValueError("v must be [B, T, H, DV] with the B, T, H of q (got %s vs %s)"
                         % (tuple(v.shape), tuple(q.shape)))
    if beta.dtype != torch.float32 or g.dtype != torch.float32:
        raise ValueError("beta and g must be float32")
    if beta.shape != q.shape[:3] or g.shape != q.shape[:3]:
        raise ValueError("beta and g must be [B, T, H]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("libgdr runs on the GPU: tensors must be on a cuda device")
    for name, t in [("q", q), ("k", k), ("v", v), ("beta", beta), ("g", g)] + list(extra):
        if t is None:
            continue
        if t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous int32 tensor on the same device")


def validate_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int) -> None:
    """Check a packed batch's cu_seqlens on the device (``gdr_validate_cu_seqlens``:
    cu[0] = 0, every later entry in [previous entry, total_tokens]) and raise
    ValueError naming the first entry that breaks it.  Synchronises with the
    current stream to read the result."""
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
            or cu_seqlens.device.type != "cuda":
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on a cuda device")
    if cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs at least two entries")
    res = torch.empty(1, dtype=torch.int32, device=cu_seqlens.device)
    stream = torch.cuda.current_stream(cu_seqlens.device).cuda_stream
    _lib.gdr_validate_cu_seqlens(cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(total_tokens),
                                 res.data_ptr(), stream)
    bad = int(res.item())
    if bad >= 0:
        raise ValueError("cu_seqlens[%d] breaks the packed-batch contract (cu[0] = 0, non-decreasing, "
                         "cu[-1] <= %d)" % (bad, total_tokens))


def _maybe_validate(cu_seqlens, total_tokens):
    # GDR_VALIDATE=1: check every packed batch's cu_seqlens before the call
    # (a synchronising debug aid; off by default)
    if cu_seqlens is not None and os.environ.get("GDR_VALIDATE", "0") == "1":
        validate_cu_seqlens(cu_seqlens, total_tokens)


def _state_shape(N, H, DK, DV, layout):
    return (N, H, DK, DV) if layout == "KV" else (N, H, DV, DK)


def chunk_gdr_fwd(q, k, v, beta, g, cu_seqlens=None, h0=None, layout="KV", scale=None,
                  output_final_state=True, save_states=False, h_store="f32", cp_segments=1):
    """Forward.  Returns (o, h_T or None, h_saved or None)."""
    _check_tensors(q, k, v, beta, g, cu_seqlens, [("h0", h0)])
    p = make_problem(q, v, cu_seqlens, layout, scale, h_store, cp_segments)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    N = p.num_seqs
    if h0 is not None and (h0.dtype != torch.float32 or tuple(h0.shape) != _state_shape(N, H, DK, DV, layout)):
        raise ValueError("h0 must be float32 %s" % (_state_shape(N, H, DK, DV, layout),))
    st = _lib.gdr_check(p)
    if st != _lib.GDR_OK:
        raise _lib.GDRError(st, _lib.last_error())
    _maybe_validate(cu_seqlens, T)
    o = torch.empty(B, T, H, DV, dtype=q.dtype, device=q.device)
    hT = torch.empty(_state_shape(N, H, DK, DV, layout), dtype=torch.float32, device=q.device) \
        if output_final_state else None
    h_saved = None
    if save_states:
        nbytes = _lib.gdr_h_saved_bytes(p)
        h_saved = torch.empty(max(nbytes, 16) // _HS_TORCH[h_store].itemsize, dtype=_HS_TORCH[h_store],
                              device=q.device)
    ws_bytes = _lib.gdr_fwd_workspace_bytes(p)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _lib.gdr_chunk_fwd(p, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(cu_seqlens), _ptr(h0),
                       _ptr(o), _ptr(hT), _ptr(h_saved), _ptr(ws), ws_bytes, stream)
    return o, hT, h_saved


GRADS = ("dq", "dk", "dv", "dbeta", "dg")


def chunk_gdr_bwd(q, k, v, beta, g, do, cu_seqlens=None, h0=None, dhT=None, h_saved=None,
                  layout="KV", scale=None, h_store="f32", need_dh0=True, cp_segments=1, need=GRADS):
    """Backward.  Returns dict(dq, dk, dv, dbeta, dg, dh0); the gradients not
    named in ``need`` (and dh0 unless ``need_dh0``) are None and not written."""
    if do.shape != v.shape or do.dtype != v.dtype:
        raise ValueError("do must match v in shape and dtype")
    _check_tensors(q, k, v, beta, g, cu_seqlens, [("h0", h0), ("do", do), ("dhT", dhT), ("h_saved", h_saved)])
    p = make_problem(q, v, cu_seqlens, layout, scale, h_store, cp_segments)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    N = p.num_seqs
    if dhT is not None and (dhT.dtype != torch.float32 or tuple(dhT.shape) != _state_shape(N, H, DK, DV, layout)):
        raise ValueError("dhT must be float32 %s" % (_state_shape(N, H, DK, DV, layout),))
    st = _lib.gdr_check(p)
    if st != _lib.GDR_OK:
        raise _lib.GDRError(st, _lib.last_error())
    if h_saved is not None and h_saved.numel() * h_saved.element_size() < _lib.gdr_h_saved_bytes(p):
        raise ValueError("h_saved is smaller than gdr_h_saved_bytes()")
    _maybe_validate(cu_seqlens, T)
    unknown = set(need) - set(GRADS)
    if unknown:
        raise ValueError("unknown gradient names %s" % sorted(unknown))
    dq = torch.empty_like(q) if "dq" in need else None
    dk = torch.empty_like(k) if "dk" in need else None
    dv = torch.empty_like(v) if "dv" in need else None
    dbeta = torch.empty_like(beta) if "dbeta" in need else None
    dg = torch.empty_like(g) if "dg" in need else None
    dh0 = torch.empty(_state_shape(N, H, DK, DV, layout), dtype=torch.float32, device=q.device) \
        if need_dh0 else None
    ws_bytes = _lib.gdr_bwd_workspace_bytes(p, h_saved is not None)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _lib.gdr_chunk_bwd(p, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(cu_seqlens), _ptr(h0),
                       _ptr(h_saved), _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta),
                       _ptr(dg), _ptr(dh0), _ptr(ws), ws_bytes, stream)
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dh0=dh0)


class ChunkGDRFunction(torch.autograd.Function):
    """Autograd over libgdr.  With ``save_states`` the forward keeps the
    per-chunk state snapshots so the backward skips their recomputation;
    without it (or when no input needs a gradient) it keeps none.  The
    backward writes only the gradients autograd asks for."""

    @staticmethod
    def forward(ctx, q, k, v, beta, g, h0, cu_seqlens, layout, scale, h_store, output_final_state,
                cp_fwd, cp_bwd, save_states):
        save = save_states and any(ctx.needs_input_grad[:6])
        o, hT, h_saved = chunk_gdr_fwd(q, k, v, beta, g, cu_seqlens=cu_seqlens, h0=h0, layout=layout,
                                       scale=scale, output_final_state=output_final_state,
                                       save_states=save, h_store=h_store, cp_segments=cp_fwd)
        ctx.save_for_backward(q, k, v, beta, g, h0, cu_seqlens, h_saved)
        ctx.layout, ctx.scale, ctx.h_store, ctx.cp_bwd = layout, scale, h_store, cp_bwd
        ctx.has_h0 = h0 is not None
        if hT is None:
            return o
        return o, hT

    @staticmethod
    def backward(ctx, do, dhT=None):
        q, k, v, beta, g, h0, cu_seqlens, h_saved = ctx.saved_tensors
        need = tuple(n for n, want in zip(GRADS, ctx.needs_input_grad[:5]) if want)
        r = chunk_gdr_bwd(q, k, v, beta, g, do.contiguous(), cu_seqlens=cu_seqlens, h0=h0,
                          dhT=None if dhT is None else dhT.contiguous(), h_saved=h_saved,
                          layout=ctx.layout, scale=ctx.scale, h_store=ctx.h_store,
                          need_dh0=ctx.has_h0 and ctx.needs_input_grad[5], cp_segments=ctx.cp_bwd,
                          need=need)
        return (r["dq"], r["dk"], r["dv"], r["dbeta"], r["dg"], r["dh0"]) + (None,) * 8


def chunk_gdr(q, k, v, beta, g, h0=None, cu_seqlens=None, layout="KV", scale=None,
              output_final_state=True, h_store="f32", cp_segments=1, cp_segments_bwd=None,
              save_states=True):
    """Chunked gated delta rule with autograd.  Returns o, or (o, h_T).
    ``cp_segments_bwd`` (default: ``cp_segments``) sets the backward's
    intra-card context parallelism independently of the forward's.
    ``save_states=False`` keeps no state snapshots between the passes (the
    backward recomputes them: less memory, one more scan)."""
    cp_bwd = cp_segments if cp_segments_bwd is None else cp_segments_bwd
    return ChunkGDRFunction.apply(q, k, v, beta, g, h0, cu_seqlens, layout, scale, h_store,
                                  output_final_state, cp_segments, cp_bwd, save_states)
