"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never touches it, and it shares no code with that path.

Two independent formulations live here:

* ``fwd`` / ``bwd`` -- the per-token recurrence and its hand-derived
  reverse-mode backward, in plain C (``gdr_oracle.c``), fp64, OpenMP over
  (sequence, head).  This is the definition every GPU result is compared with.
* ``chunk_fwd`` -- the chunk-wise form of the same forward (chunk-local
  cumulative decay, the strictly-lower-triangular system ``(I + A) T = I``,
  the W/U transform, the inter-chunk state update), written in NumPy with
  library matmul and inverse as steps.  It exists to pin the recurrence
  (the two must agree to rounding) and to expose per-chunk intermediates.

The operator is the "chunked gated delta rule" named by FlashQLA PR #34
("SM120/121 : Add support for fused backward kernel", section "Summary"); the
pages give no formula, so the recurrence is the standard gated delta rule:
``S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T``,
``o_t = scale S_t q_t``.  State layouts KV (``h = S^T``, [DK, DV]) and VK
(``S``, [DV, DK]) are the "KV/VK state layouts" of the same page, section
"Current status"; the layout flag only changes memory order.

Tensor conventions (NumPy arrays, any float dtype; converted to float64):
  q, k: [B, T, H, DK]; v, do: [B, T, H, DV]; beta, g: [B, T, H];
  cu_seqlens: int array [N+1] (then B must be 1 and sequences are packed
  along T); states h0 / hT / dhT / dh0: [N, H, DK, DV] (KV) or
  [N, H, DV, DK] (VK).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (host only, fp64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _setup(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.gdr_oracle_fwd.argtypes = [ctypes.c_int, ip, ip, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_double] + [dp] * 8 + [ctypes.c_int]
    lib.gdr_oracle_fwd.restype = ctypes.c_int
    lib.gdr_oracle_bwd.argtypes = [ctypes.c_int, ip, ip, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_double] + [dp] * 14 + [ctypes.c_int]
    lib.gdr_oracle_bwd.restype = ctypes.c_int
    lib.gdr_oracle_max_threads.argtypes = []
    lib.gdr_oracle_max_threads.restype = ctypes.c_int
    return lib


def load_variant(path: str):
    """Load another build of the C oracle (used by the tests that plant
    mistakes in a copy of the source to show the pins catch them)."""
    return _setup(ctypes.CDLL(path))


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = _setup(ctypes.CDLL(_LIB))
    return _lib


def max_threads() -> int:
    return int(_load().gdr_oracle_max_threads())


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: read its values on the host
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _segments(B, T, cu_seqlens):
    if cu_seqlens is None:
        start = np.arange(B, dtype=np.int64) * T
        length = np.full(B, T, dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
        assert B == 1, "packed (varlen) input must have batch 1"
        start = cu[:-1].copy()
        length = (cu[1:] - cu[:-1]).copy()
        assert np.all(length >= 0) and cu[0] == 0 and cu[-1] <= T
    return np.ascontiguousarray(start), np.ascontiguousarray(length)


def _to_vk(h, layout):
    if h is None:
        return None
    h = _f64(h)
    return np.ascontiguousarray(np.swapaxes(h, -1, -2)) if layout == "KV" else h


def _from_vk(s, layout):
    return np.ascontiguousarray(np.swapaxes(s, -1, -2)) if layout == "KV" else s


def fwd(q, k, v, beta, g, cu_seqlens=None, h0=None, scale=None, layout="VK",
        nthreads: int = 0, lib=None):
    """Per-token recurrent forward.  Returns (o [B,T,H,DV], hT in `layout`)."""
    assert layout in ("KV", "VK")
    q, k, v, beta, g = (_f64(x) for x in (q, k, v, beta, g))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if scale is None:
        scale = DK ** -0.5
    start, length = _segments(B, T, cu_seqlens)
    N = len(start)
    s0 = _to_vk(h0, layout)
    o = np.zeros((B, T, H, DV))
    hT = np.zeros((N, H, DV, DK))
    ip = ctypes.POINTER(ctypes.c_int64)
    rc = (lib or _load()).gdr_oracle_fwd(N, start.ctypes.data_as(ip), length.ctypes.data_as(ip), H, DK, DV,
                                float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                _ptr(s0), _ptr(o), _ptr(hT), int(nthreads))
    if rc != 0:
        raise MemoryError("oracle forward: allocation failed")
    return o, _from_vk(hT, layout)


def bwd(q, k, v, beta, g, do, cu_seqlens=None, h0=None, dhT=None, scale=None,
        layout="VK", nthreads: int = 0, lib=None):
    """Hand-derived reverse-mode backward of the recurrence.

    Returns a dict with dq, dk, dv, dbeta, dg and dh0 (dh0 in `layout`)."""
    assert layout in ("KV", "VK")
    q, k, v, beta, g, do = (_f64(x) for x in (q, k, v, beta, g, do))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if scale is None:
        scale = DK ** -0.5
    start, length = _segments(B, T, cu_seqlens)
    N = len(start)
    s0 = _to_vk(h0, layout)
    ds = _to_vk(dhT, layout)
    out = dict(dq=np.zeros((B, T, H, DK)), dk=np.zeros((B, T, H, DK)),
               dv=np.zeros((B, T, H, DV)), dbeta=np.zeros((B, T, H)), dg=np.zeros((B, T, H)))
    dh0 = np.zeros((N, H, DV, DK))
    ip = ctypes.POINTER(ctypes.c_int64)
    rc = (lib or _load()).gdr_oracle_bwd(N, start.ctypes.data_as(ip), length.ctypes.data_as(ip), H, DK,
                                DV, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                _ptr(s0), _ptr(do), _ptr(ds), _ptr(out["dq"]), _ptr(out["dk"]),
                                _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dg"]), _ptr(dh0),
                                int(nthreads))
    if rc != 0:
        raise MemoryError("oracle backward: allocation failed")
    out["dh0"] = _from_vk(dh0, layout)
    return out


def chunk_fwd(q, k, v, beta, g, cu_seqlens=None, h0=None, scale=None, layout="VK",
              chunk: int = 64, keep: bool = False):
    """Chunk-wise forward of the same recurrence (NumPy, fp64).

    Per sequence and head, chunks of `chunk` tokens restart at each sequence
    start; the last chunk may be partial.  Inside a chunk of C' rows (state h
    in KV form at the chunk start):
      gamma = inclusive cumsum of g                   (cumulative log-decay)
      Gam[r,s] = exp(gamma_r - gamma_s) for s <= r, else 0
      A = strictly_lower(diag(beta) K K^T * Gam)
      T = (I + A)^-1
      W = T diag(beta * exp(gamma)) K,   U = T diag(beta) V
      Delta = U - W h                                 (new values)
      O = scale * (diag(exp(gamma)) Q h + (Q K^T * Gam) Delta)
      h <- exp(gamma_last) h + (diag(exp(gamma_last - gamma)) K)^T Delta
    Returns (o, hT) and, if keep, a list of per-(sequence, head) dicts with
    the per-chunk intermediates (gamma, T, W, U, h at chunk start, Delta).
    """
    q, k, v, beta, g = (_f64(x) for x in (q, k, v, beta, g))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if scale is None:
        scale = DK ** -0.5
    start, length = _segments(B, T, cu_seqlens)
    N = len(start)
    s0 = _to_vk(h0, layout)
    qf, kf, vf = (x.reshape(B * T, H, -1) for x in (q, k, v))
    bf, gf = beta.reshape(B * T, H), g.reshape(B * T, H)
    o = np.zeros((B * T, H, DV))
    hT = np.zeros((N, H, DV, DK))
    inter = []
    for n in range(N):
        for hd in range(H):
            h = np.zeros((DK, DV)) if s0 is None else s0[n, hd].T.copy()
            rec = []
            t0, L = int(start[n]), int(length[n])
            for c0 in range(0, L, chunk):
                rows = np.arange(t0 + c0, t0 + min(c0 + chunk, L))
                Q, K, V = qf[rows, hd], kf[rows, hd], vf[rows, hd]
                bt, gt = bf[rows, hd], gf[rows, hd]
                Cp = len(rows)
                gam = np.cumsum(gt)
                diff = gam[:, None] - gam[None, :]
                mask = np.tril(np.ones((Cp, Cp), dtype=bool))
                Gam = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
                A = np.tril(bt[:, None] * (K @ K.T) * Gam, -1)
                Tm = np.linalg.inv(np.eye(Cp) + A)
                W = Tm @ ((bt * np.exp(gam))[:, None] * K)
                U = Tm @ (bt[:, None] * V)
                Delta = U - W @ h
                P = (Q @ K.T) * Gam
                o[rows, hd] = scale * ((np.exp(gam)[:, None] * Q) @ h + P @ Delta)
                if keep:
                    rec.append(dict(gamma=gam, T=Tm, W=W, U=U, h=h.copy(), Delta=Delta))
                Kt = np.exp(gam[-1] - gam)[:, None] * K
                h = np.exp(gam[-1]) * h + Kt.T @ Delta
            hT[n, hd] = h.T
            if keep:
                inter.append(rec)
    o = o.reshape(B, T, H, DV)
    res = (o, _from_vk(hT, layout))
    return res + (inter,) if keep else res
