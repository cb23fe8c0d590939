"""ctypes binding of libgdr's C ABI (include/libgdr.h), same names.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgdr.so.  Loading fails loudly if the library has not been
built -- there is no fallback of any kind.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdr.so")
# race-test build: same kernels, barriers that can delay chosen waves
DELAY_LIB_PATH = os.path.join(HERE, "libgdr_delay.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_WORKSPACE, GDR_ERR_HIP = range(5)
GDR_F32, GDR_BF16, GDR_F16 = 0, 1, 2
GDR_LAYOUT_KV, GDR_LAYOUT_VK = 0, 1

# every function the header declares, for the export check
EXPORTS = ("gdr_check", "gdr_fwd_workspace_bytes", "gdr_bwd_workspace_bytes", "gdr_h_saved_bytes",
           "gdr_chunk_fwd", "gdr_chunk_bwd", "gdr_chunk_fwd_noalloc", "gdr_validate_cu_seqlens",
           "gdr_set_kernel_timers", "gdr_status_string", "gdr_last_error", "gdr_version")
# include/gdr_rmsnorm.h: the fused RMSNorm backward and its reduction modes
RMSNORM_EXPORTS = ("gdr_rmsnorm_bwd_workspace_bytes", "gdr_rmsnorm_bwd")
GDR_REDUCE_FIXED, GDR_REDUCE_ATOMIC, GDR_REDUCE_SEPARATE = 0, 1, 2
# size of the static workspace of gdr_chunk_fwd_noalloc (GDR_NOALLOC_SCRATCH_BYTES)
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20
KERNELS = ("plan", "wy", "scan_fwd", "scan_bwd", "grad", "cp_scan_fwd", "cp_chain_fwd", "cp_scan_bwd",
           "cp_chain_bwd")


class gdr_problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("varlen", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("h_store_dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("cp_segments", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class GDRError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (status_string(status), message))
        self.status = status


_lock = threading.RLock()
_lib = None        # the library the calls below use by default
_libs = {}         # every library opened, by path
_override = None   # the library selected by using(), if any


def _open(path: str):
    with _lock:
        if path in _libs:
            return _libs[path]
        if not os.path.exists(path):
            raise RuntimeError(
                "%s is not built. Build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` or "
                "`python chunked_gated_delta_02_amd/build.py`." % path)
        # RTLD_LOCAL: a second build of the library (the race-test one) keeps
        # its own kernels and host code
        lib = ctypes.CDLL(path, mode=os.RTLD_LOCAL)
        P = ctypes.POINTER(gdr_problem)
        vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.gdr_check.argtypes = [P]
        lib.gdr_check.restype = ctypes.c_int
        lib.gdr_fwd_workspace_bytes.argtypes = [P]
        lib.gdr_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_bwd_workspace_bytes.argtypes = [P, ctypes.c_int]
        lib.gdr_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_h_saved_bytes.argtypes = [P]
        lib.gdr_h_saved_bytes.restype = ctypes.c_size_t
        lib.gdr_chunk_fwd.argtypes = [P, vp, vp, vp, fp, fp, ip, fp, vp, fp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_fwd.restype = ctypes.c_int
        lib.gdr_chunk_bwd.argtypes = [P, vp, vp, vp, fp, fp, ip, fp, vp, vp, fp, vp, vp, vp, fp, fp, fp,
                                      vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_bwd.restype = ctypes.c_int
        lib.gdr_chunk_fwd_noalloc.argtypes = [P, vp, vp, vp, fp, fp, ip, fp, vp, fp, vp, vp]
        lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
        ci = ctypes.c_int
        lib.gdr_validate_cu_seqlens.argtypes = [ip, ci, ci, ip, vp]
        lib.gdr_validate_cu_seqlens.restype = ci
        lib.gdr_rmsnorm_bwd_workspace_bytes.argtypes = [ci, ci, ci]
        lib.gdr_rmsnorm_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_rmsnorm_bwd.argtypes = [ci, ci, ci, vp, fp, vp, fp, ctypes.c_float, vp, fp, ci, vp,
                                        ctypes.c_size_t, vp]
        lib.gdr_rmsnorm_bwd.restype = ctypes.c_int
        lib.gdr_set_kernel_timers.argtypes = [ctypes.c_void_p]
        lib.gdr_set_kernel_timers.restype = ctypes.c_int
        lib.gdr_status_string.argtypes = [ctypes.c_int]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_last_error.argtypes = []
        lib.gdr_last_error.restype = ctypes.c_char_p
        lib.gdr_version.argtypes = []
        lib.gdr_version.restype = ctypes.c_int
        if hasattr(lib, "gdr_debug_set_delay"):
            lib.gdr_debug_set_delay.argtypes = [ctypes.c_int] * 4
            lib.gdr_debug_set_delay.restype = ctypes.c_int
        _libs[path] = lib
        return lib


def load(path: str = LIB_PATH):
    """Load libgdr.so (or, on the first call, the build at `path`); raises if
    it is missing (build it first)."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = _open(path)
        return _lib


def _h():
    return _override if _override is not None else load()


@contextlib.contextmanager
def using(path: str):
    """Route every call made inside the block to the build at `path` (the
    race-test build DELAY_LIB_PATH in the tests).  The switch is process-wide:
    calls from other threads during the block go to that build too."""
    global _override
    lib = _open(path)
    prev = _override
    _override = lib
    try:
        yield lib
    finally:
        _override = prev


def status_string(status: int) -> str:
    return _h().gdr_status_string(int(status)).decode()


def last_error() -> str:
    return _h().gdr_last_error().decode()


def _raise_on(status: int) -> int:
    if status != GDR_OK:
        raise GDRError(status, last_error())
    return status


def gdr_check(p: gdr_problem) -> int:
    return _h().gdr_check(ctypes.byref(p))


def gdr_fwd_workspace_bytes(p: gdr_problem) -> int:
    return _h().gdr_fwd_workspace_bytes(ctypes.byref(p))


def gdr_bwd_workspace_bytes(p: gdr_problem, have_h_saved: bool) -> int:
    return _h().gdr_bwd_workspace_bytes(ctypes.byref(p), int(bool(have_h_saved)))


def gdr_h_saved_bytes(p: gdr_problem) -> int:
    return _h().gdr_h_saved_bytes(ctypes.byref(p))


def gdr_version() -> int:
    return _h().gdr_version()


def gdr_chunk_fwd(p, q, k, v, beta, g, cu_seqlens, h0, o, hT, h_saved, ws, ws_bytes, stream,
                  check=True) -> int:
    """Raw call; all tensor arguments are integer device addresses (0 = NULL)."""
    st = _h().gdr_chunk_fwd(ctypes.byref(p), q, k, v, beta, g, cu_seqlens or None, h0 or None, o,
                              hT or None, h_saved or None, ws or None, ws_bytes, stream or None)
    return _raise_on(st) if check else st


def gdr_chunk_fwd_noalloc(p, q, k, v, beta, g, cu_seqlens, h0, o, hT, h_saved, stream, check=True) -> int:
    """Raw call of the allocation-free forward (the library's static
    workspace); all tensor arguments are integer device addresses (0 = NULL)."""
    st = _h().gdr_chunk_fwd_noalloc(ctypes.byref(p), q, k, v, beta, g, cu_seqlens or None, h0 or None, o,
                                      hT or None, h_saved or None, stream or None)
    return _raise_on(st) if check else st


def gdr_validate_cu_seqlens(cu_seqlens, num_seqs, total_tokens, result, stream, check=True) -> int:
    """Raw call: launches the device check of a packed batch's cu_seqlens;
    the kernel writes the first violating index (or -1) to the device int at
    `result`.  Addresses are integers (0 = NULL)."""
    st = _h().gdr_validate_cu_seqlens(cu_seqlens or None, int(num_seqs), int(total_tokens), result or None,
                                      stream or None)
    return _raise_on(st) if check else st


def gdr_rmsnorm_bwd_workspace_bytes(M: int, N: int, mode: int) -> int:
    return _h().gdr_rmsnorm_bwd_workspace_bytes(int(M), int(N), int(mode))


def gdr_rmsnorm_bwd(M, N, io_dtype, x, w, dy, rstd, eps, dx, dw, mode, ws, ws_bytes, stream,
                    check=True) -> int:
    """Raw call (include/gdr_rmsnorm.h); tensor arguments are integer device
    addresses (0 = NULL)."""
    st = _h().gdr_rmsnorm_bwd(int(M), int(N), int(io_dtype), x, w, dy, rstd or None, float(eps), dx, dw,
                              int(mode), ws or None, ws_bytes, stream or None)
    return _raise_on(st) if check else st


def gdr_chunk_bwd(p, q, k, v, beta, g, cu_seqlens, h0, h_saved, dO, dhT, dq, dk, dv, dbeta, dg,
                  dh0, ws, ws_bytes, stream, check=True) -> int:
    """Raw call; all tensor arguments are integer device addresses (0 = NULL)."""
    st = _h().gdr_chunk_bwd(ctypes.byref(p), q, k, v, beta, g, cu_seqlens or None, h0 or None,
                              h_saved or None, dO, dhT or None, dq, dk, dv, dbeta, dg, dh0 or None,
                              ws or None, ws_bytes, stream or None)
    return _raise_on(st) if check else st


def gdr_set_kernel_timers(events) -> int:
    """events: None, or a sequence of 2 * len(KERNELS) hipEvent_t handles
    (ints, 0 = not timed) -- (start, stop) per kernel id."""
    if events is None:
        return _raise_on(_h().gdr_set_kernel_timers(None))
    assert len(events) == 2 * len(KERNELS)
    arr = (ctypes.c_void_p * len(events))(*[e or None for e in events])
    return _raise_on(_h().gdr_set_kernel_timers(arr))


def gdr_debug_set_delay(wave: int, mod: int, iters: int, salt: int = 0) -> int:
    """Barrier delays of the race-test build (include/libgdr_debug.h); only
    that build exports it."""
    lib = _h()
    if not hasattr(lib, "gdr_debug_set_delay"):
        raise RuntimeError("gdr_debug_set_delay: only the race-test build (libgdr_delay.so) exports it")
    return _raise_on(lib.gdr_debug_set_delay(int(wave), int(mod), int(iters), int(salt)))
