"""PyTorch-facing wrapper of libgdr's fused RMSNorm backward
(include/gdr_rmsnorm.h): allocation of dx, dw and the workspace with torch on
the current stream, argument marshalling only -- the computation runs in the
library's HIP kernels.

The operator is the RMSNorm backward whose weight-gradient partials
Dao-AILab/quack PR #101 ("Rmsnorm backward fusing sum") reduces inside the
backward kernel; ``mode`` picks how that cross-workgroup reduction is done
(the determinism question of the same page's review thread):

* ``"fixed"`` (default): in-kernel, fixed order, bitwise reproducible;
* ``"atomic"``: in-kernel floating-point atomics, order not fixed;
* ``"separate"``: a second kernel sums the partials in a fixed order.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

MODES = {"fixed": _lib.GDR_REDUCE_FIXED, "atomic": _lib.GDR_REDUCE_ATOMIC,
         "separate": _lib.GDR_REDUCE_SEPARATE}
_IO = {torch.bfloat16: _lib.GDR_BF16, torch.float32: _lib.GDR_F32}


def workspace(M: int, N: int, mode: str = "fixed", device=None) -> Optional[torch.Tensor]:
    """A workspace for (M, N, mode), zeroed as the fixed-order mode's arrival
    counters require (every call leaves them zero again, so it can be kept
    and reused by later calls on the same stream)."""
    nb = _lib.gdr_rmsnorm_bwd_workspace_bytes(M, N, MODES[mode])
    if nb == 0:
        return None
    return torch.zeros(nb, dtype=torch.uint8, device=device)


def rmsnorm_bwd(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rstd: Optional[torch.Tensor] = None,
                eps: float = 1e-6, dw: Optional[torch.Tensor] = None, mode: str = "fixed",
                ws: Optional[torch.Tensor] = None):
    """Returns (dx, dw).  x, dy: [M, N] bf16 or fp32 on the GPU; w: [N] fp32;
    rstd: [M] fp32 (the forward's 1/rms; None = recomputed with eps).  dw, if
    given, is accumulated into (dw += ...); otherwise a zeroed one is made."""
    if mode not in MODES:
        raise ValueError("mode must be one of %s" % sorted(MODES))
    if x.dim() != 2 or dy.shape != x.shape or dy.dtype != x.dtype or x.dtype not in _IO:
        raise ValueError("x and dy must be [M, N] tensors of one dtype, bfloat16 or float32")
    M, N = x.shape
    if w.shape != (N,) or w.dtype != torch.float32:
        raise ValueError("w must be float32 [N]")
    if rstd is not None and (rstd.shape != (M,) or rstd.dtype != torch.float32):
        raise ValueError("rstd must be float32 [M]")
    if x.device.type != "cuda":
        raise ValueError("libgdr runs on the GPU: tensors must be on a cuda device")
    for name, t in (("x", x), ("w", w), ("dy", dy), ("rstd", rstd), ("dw", dw), ("ws", ws)):
        if t is not None and (t.device != x.device or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous tensor on %s" % (name, x.device))
    if dw is None:
        dw = torch.zeros(N, dtype=torch.float32, device=x.device)
    elif dw.shape != (N,) or dw.dtype != torch.float32:
        raise ValueError("dw must be float32 [N]")
    if ws is None:
        ws = workspace(M, N, mode, x.device)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    dx = torch.empty_like(x)
    P = lambda t: 0 if t is None else t.data_ptr()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _lib.gdr_rmsnorm_bwd(M, N, _IO[x.dtype], P(x), P(w), P(dy), P(rstd), eps, P(dx), P(dw), MODES[mode],
                         P(ws), nb, stream)
    return dx, dw
