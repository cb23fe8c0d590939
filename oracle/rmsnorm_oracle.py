"""fp64 CPU oracle for the RMSNorm backward -- TEST INFRASTRUCTURE ONLY.

Only the tests and the CPU-baseline leg of ``bench.py`` may import this
module.  The product path (the HIP library and its Python binding) never
touches it, and it shares no code with that path.

The operator is the RMSNorm backward whose weight-gradient partial sums
Dao-AILab/quack PR #101 ("Rmsnorm backward fusing sum", description) folds
into the backward kernel itself.  The page gives no formula; the forward is
the standard RMSNorm of each row x (length N) with weight w and epsilon eps:

    r = (mean_j x_j^2 + eps)^(-1/2),   y_j = w_j x_j r.

For a cotangent dy, with xhat = r x, differentiating by hand:

    d r / d x_k = -r^3 x_k / N
    dx_k = r (w_k dy_k) - x_k r^3 (1/N) sum_j w_j dy_j x_j
         = r (w_k dy_k - xhat_k mean_j(w_j dy_j xhat_j))
    dw_j = sum over rows of dy_j xhat_j

When the forward's r is passed in (``rstd``) it is used as is; otherwise it
is computed from x and eps.  Arrays: x, dy [M, N]; w [N]; rstd [M].
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: read its values on the host
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def rstd(x, eps: float):
    """r = 1 / sqrt(mean_j x_j^2 + eps) per row."""
    x = _f64(x)
    return 1.0 / np.sqrt((x * x).mean(axis=-1) + eps)


def forward(x, w, eps: float):
    """y = w * x * r (row-wise); returns (y, r)."""
    x, w = _f64(x), _f64(w)
    r = rstd(x, eps)
    return w[None, :] * x * r[:, None], r


def backward(x, w, dy, r=None, eps: float = 0.0):
    """Gradients (dx, dw) of L = <dy, y>, y = RMSNorm(x; w, eps).  `r` is the
    forward's 1/rms per row; None = computed from x and eps."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    r = rstd(x, eps) if r is None else _f64(r)
    M, N = x.shape
    xhat = x * r[:, None]
    wdy = w[None, :] * dy
    c = (wdy * xhat).sum(axis=1) / N            # mean_j(w_j dy_j xhat_j) per row
    dx = r[:, None] * (wdy - xhat * c[:, None])
    dw = (dy * xhat).sum(axis=0)
    return dx, dw


def backward_rows(x, w, dy, r=None, eps: float = 0.0):
    """The same gradients taken one row at a time with scalar loops (small
    inputs only): dw accumulated row after row, as its definition reads."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    M, N = x.shape
    dx = np.zeros((M, N))
    dw = np.zeros(N)
    for m in range(M):
        ss = 0.0
        for j in range(N):
            ss += x[m, j] * x[m, j]
        rm = 1.0 / np.sqrt(ss / N + eps) if r is None else float(_f64(r)[m])
        acc = 0.0
        for j in range(N):
            acc += w[j] * dy[m, j] * x[m, j] * rm
        cm = acc / N
        for j in range(N):
            xh = x[m, j] * rm
            dx[m, j] = rm * (w[j] * dy[m, j] - xh * cm)
            dw[j] += dy[m, j] * xh
    return dx, dw
