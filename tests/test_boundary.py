"""The C-ABI boundary on the host: exports, argument validation, workspace
sizing.  No call here reaches a GPU -- every error path returns before any
launch, which is what these tests check."""
import ctypes
import os
import re

import pytest

from chunked_gated_delta_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgdr.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from chunked_gated_delta_02_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_race_build_exports_the_delay_hook_and_production_does_not(lib):
    # libgdr_delay.so: every libgdr.h function plus gdr_debug_set_delay
    # (include/libgdr_debug.h); libgdr.so: not the hook
    assert not hasattr(lib, "gdr_debug_set_delay")
    if not os.path.exists(_lib.DELAY_LIB_PATH):
        from chunked_gated_delta_02_amd import build
        build.build()
    with _lib.using(_lib.DELAY_LIB_PATH) as d:
        for n in _lib.EXPORTS + ("gdr_debug_set_delay",):
            assert ctypes.cast(getattr(d, n), ctypes.c_void_p).value, n
        text = open(os.path.join(ROOT, "include", "libgdr_debug.h")).read()
        assert "gdr_debug_set_delay(" in text
        # settings out of range are refused on the host, before any device call
        for args in ((8, 1, 1), (-2, 1, 1), (0, 0, 1), (0, 1, -1), (0, 1, 65)):
            with pytest.raises(_lib.GDRError) as e:
                _lib.gdr_debug_set_delay(*args)
            assert e.value.status == _lib.GDR_ERR_INVALID_ARG
    with pytest.raises(RuntimeError):
        _lib.gdr_debug_set_delay(0, 1, 0)


def good(**kw):
    p = _lib.gdr_problem()
    p.batch, p.seqlen, p.num_seqs, p.varlen, p.heads = 2, 4096, 2, 0, 16
    p.dk, p.dv, p.chunk = 128, 128, 64
    p.io_dtype, p.h_store_dtype, p.layout, p.cp_segments, p.scale = _lib.GDR_BF16, _lib.GDR_F32, 0, 1, 0.0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_valid_problems(lib):
    assert _lib.gdr_check(good()) == _lib.GDR_OK
    assert _lib.gdr_check(good(io_dtype=_lib.GDR_F32, dk=64, dv=64)) == _lib.GDR_OK
    assert _lib.gdr_check(good(varlen=1, batch=1, num_seqs=8, seqlen=30000)) == _lib.GDR_OK
    assert _lib.gdr_check(good(dv=256, h_store_dtype=_lib.GDR_F16)) == _lib.GDR_OK
    assert _lib.gdr_check(good(seqlen=0)) == _lib.GDR_OK


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0, num_seqs=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(seqlen=-1), _lib.GDR_ERR_INVALID_ARG),
    (dict(heads=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(num_seqs=3), _lib.GDR_ERR_INVALID_ARG),
    (dict(varlen=1), _lib.GDR_ERR_INVALID_ARG),          # batch 2 with varlen
    (dict(varlen=1, batch=1, num_seqs=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(varlen=1, batch=1, num_seqs=100000), _lib.GDR_ERR_UNSUPPORTED),
    (dict(varlen=2), _lib.GDR_ERR_INVALID_ARG),
    (dict(chunk=32), _lib.GDR_ERR_UNSUPPORTED),
    (dict(dk=96), _lib.GDR_ERR_UNSUPPORTED),
    (dict(dv=100), _lib.GDR_ERR_UNSUPPORTED),
    (dict(dv=1024), _lib.GDR_ERR_UNSUPPORTED),
    (dict(io_dtype=_lib.GDR_F16), _lib.GDR_ERR_UNSUPPORTED),
    (dict(io_dtype=7), _lib.GDR_ERR_UNSUPPORTED),
    (dict(h_store_dtype=9), _lib.GDR_ERR_INVALID_ARG),
    (dict(io_dtype=_lib.GDR_F32, h_store_dtype=_lib.GDR_F16), _lib.GDR_ERR_UNSUPPORTED),
    (dict(layout=2), _lib.GDR_ERR_INVALID_ARG),
    (dict(cp_segments=0), _lib.GDR_ERR_INVALID_ARG),
    # a chunk's rows of every head must stay addressable with 32-bit byte
    # offsets: 64 x H x max(dk, dv) x element size < 2^31
    (dict(io_dtype=_lib.GDR_F32, dv=512, heads=16384), _lib.GDR_ERR_UNSUPPORTED),
    (dict(dv=512, heads=32768, seqlen=64), _lib.GDR_ERR_UNSUPPORTED),
])
def test_invalid_problems(lib, kw, status):
    assert _lib.gdr_check(good(**kw)) == status
    assert _lib.gdr_fwd_workspace_bytes(good(**kw)) == 0
    assert _lib.last_error() != ""


def test_largest_addressable_head_count(lib):
    # 64 x 16383 x 512 x 4 bytes is just below 2^31
    assert _lib.gdr_check(good(io_dtype=_lib.GDR_F32, dv=512, heads=16383, seqlen=64)) == _lib.GDR_OK
    assert _lib.gdr_check(good(dv=512, heads=32767, seqlen=64)) == _lib.GDR_OK


def test_null_problem(lib):
    assert lib.gdr_check(None) == _lib.GDR_ERR_INVALID_ARG


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced: calls fail before any launch


def fwd_args(p, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, cu=0, h0=0, o=FAKE, hT=0, hs=0,
             ws=FAKE, ws_bytes=_lib.gdr_fwd_workspace_bytes(p), stream=0)
    a.update(kw)
    return a


def call_fwd(p, a):
    return _lib.gdr_chunk_fwd(p, a["q"], a["k"], a["v"], a["beta"], a["g"], a["cu"], a["h0"], a["o"],
                              a["hT"], a["hs"], a["ws"], a["ws_bytes"], a["stream"], check=False)


@pytest.mark.parametrize("field", ["q", "k", "v", "beta", "g", "o"])
def test_fwd_null_required_pointer(lib, field):
    p = good()
    assert call_fwd(p, fwd_args(p, **{field: 0})) == _lib.GDR_ERR_INVALID_ARG


def test_fwd_misaligned_pointer(lib):
    p = good()
    assert call_fwd(p, fwd_args(p, v=FAKE + 2)) == _lib.GDR_ERR_INVALID_ARG
    assert call_fwd(p, fwd_args(p, h0=FAKE + 8)) == _lib.GDR_ERR_INVALID_ARG


def test_fwd_workspace_too_small_or_missing(lib):
    p = good()
    need = _lib.gdr_fwd_workspace_bytes(p)
    assert call_fwd(p, fwd_args(p, ws_bytes=need - 1)) == _lib.GDR_ERR_WORKSPACE
    assert call_fwd(p, fwd_args(p, ws=0)) == _lib.GDR_ERR_WORKSPACE


def test_fwd_cu_seqlens_consistency(lib):
    p = good()
    assert call_fwd(p, fwd_args(p, cu=FAKE)) == _lib.GDR_ERR_INVALID_ARG
    pv = good(varlen=1, batch=1, num_seqs=4)
    assert call_fwd(pv, fwd_args(pv)) == _lib.GDR_ERR_INVALID_ARG


def test_context_parallel_limits_and_workspace(lib):
    assert _lib.gdr_check(good(cp_segments=4)) == _lib.GDR_OK
    assert _lib.gdr_check(good(cp_segments=1024)) == _lib.GDR_OK
    assert _lib.gdr_check(good(cp_segments=1025)) == _lib.GDR_ERR_UNSUPPORTED
    # CP needs the segment summaries [DK x (DK + DV)] and hand-off states
    # [DK x DV] (fp32) per (segment, sequence, head) on top of the plain plan
    p1, p4 = good(), good(cp_segments=4)
    extra = 4 * p4.num_seqs * p4.heads * p4.dk * (2 * p4.dv + p4.dk) * 4
    for f in (lambda p: _lib.gdr_fwd_workspace_bytes(p), lambda p: _lib.gdr_bwd_workspace_bytes(p, True)):
        assert extra <= f(p4) - f(p1) <= extra + 512
    # the saved snapshots do not depend on the segmentation
    assert _lib.gdr_h_saved_bytes(p1) == _lib.gdr_h_saved_bytes(p4)


def test_bwd_validation(lib):
    p = good()
    ws = _lib.gdr_bwd_workspace_bytes(p, False)
    args = [FAKE] * 5 + [0, 0, 0, FAKE, 0] + [FAKE] * 5 + [0]
    st = _lib.gdr_chunk_bwd(p, *args, FAKE, ws - 1, 0, check=False)
    assert st == _lib.GDR_ERR_WORKSPACE
    bad = list(args)
    bad[8] = 0  # dO
    assert _lib.gdr_chunk_bwd(p, *bad, FAKE, ws, 0, check=False) == _lib.GDR_ERR_INVALID_ARG


def test_workspace_sizes(lib):
    p = good()
    f = _lib.gdr_fwd_workspace_bytes(p)
    b0 = _lib.gdr_bwd_workspace_bytes(p, False)
    b1 = _lib.gdr_bwd_workspace_bytes(p, True)
    hs = _lib.gdr_h_saved_bytes(p)
    nchunks = 2 * 64
    assert hs == nchunks * 16 * 128 * 128 * 4
    assert b0 - b1 >= hs
    assert f > 0 and b1 > 0
    # the forward keeps snapshots only in the caller's h_saved: its workspace
    # does not depend on the snapshot dtype
    assert _lib.gdr_fwd_workspace_bytes(good(h_store_dtype=_lib.GDR_F16)) == f
    assert _lib.gdr_h_saved_bytes(good(h_store_dtype=_lib.GDR_F16)) == hs // 2
    # packed batches: chunk slots bounded by ceil(T/64) + N without reading cu_seqlens
    pv = good(varlen=1, batch=1, num_seqs=8, seqlen=1000)
    assert _lib.gdr_h_saved_bytes(pv) == (16 + 8) * 16 * 128 * 128 * 4
    assert _lib.gdr_fwd_workspace_bytes(good(seqlen=8192)) > f


def test_status_strings_and_version(lib):
    assert _lib.status_string(_lib.GDR_OK) == "GDR_OK"
    assert _lib.status_string(_lib.GDR_ERR_WORKSPACE) == "GDR_ERR_WORKSPACE"
    assert _lib.gdr_version() >= 100


# ---------------------------------------------------------------------------
# the fused RMSNorm backward (include/gdr_rmsnorm.h): exports and host checks

def test_rmsnorm_header_functions_are_exported(lib):
    text = open(os.path.join(ROOT, "include", "gdr_rmsnorm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))
    assert set(names) == set(_lib.RMSNORM_EXPORTS), names
    for n in names:
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value, n


def _rn(M=64, N=256, io=None, mode=None, ws=FAKE, ws_bytes=None, **kw):
    io = _lib.GDR_BF16 if io is None else io
    mode = _lib.GDR_REDUCE_FIXED if mode is None else mode
    a = dict(x=FAKE, w=FAKE, dy=FAKE, rstd=0, eps=1e-6, dx=FAKE, dw=FAKE)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = _lib.gdr_rmsnorm_bwd_workspace_bytes(M, N, mode)
    return _lib.gdr_rmsnorm_bwd(M, N, io, a["x"], a["w"], a["dy"], a["rstd"], a["eps"], a["dx"], a["dw"],
                                mode, ws, ws_bytes, 0, check=False)


def test_rmsnorm_workspace_sizes(lib):
    # fixed: 512 B of counters + G partials + ceil(G/32) group sums (fp32);
    # separate: counters + partials; atomic: none.  G = ceil(M/16), at most
    # 256 (512 for 1024 < N <= 2048)
    f = _lib.gdr_rmsnorm_bwd_workspace_bytes
    assert f(64, 256, _lib.GDR_REDUCE_ATOMIC) == 0
    assert f(64, 256, _lib.GDR_REDUCE_SEPARATE) == 512 + 4 * 256 * 4
    assert f(64, 256, _lib.GDR_REDUCE_FIXED) == 512 + 4 * 256 * 4 + 1 * 256 * 4
    assert f(65536, 8192, _lib.GDR_REDUCE_FIXED) == 512 + 256 * 8192 * 4 + 8 * 8192 * 4
    assert f(65536, 2048, _lib.GDR_REDUCE_FIXED) == 512 + 512 * 2048 * 4 + 16 * 2048 * 4
    assert f(64, 12, _lib.GDR_REDUCE_FIXED) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(N=12), _lib.GDR_ERR_UNSUPPORTED),            # not a multiple of 8
    (dict(N=8200), _lib.GDR_ERR_UNSUPPORTED),          # wider than 8192
    (dict(M=-1), _lib.GDR_ERR_UNSUPPORTED),
    (dict(io=_lib.GDR_F16), _lib.GDR_ERR_UNSUPPORTED),
    (dict(mode=3), _lib.GDR_ERR_INVALID_ARG),
    (dict(eps=-1.0), _lib.GDR_ERR_INVALID_ARG),        # rstd not given: eps must be >= 0
    (dict(dx=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(w=FAKE + 4), _lib.GDR_ERR_INVALID_ARG),      # misaligned
    (dict(ws=0), _lib.GDR_ERR_WORKSPACE),
    (dict(ws_bytes=100), _lib.GDR_ERR_WORKSPACE),
])
def test_rmsnorm_invalid_arguments_return_before_any_launch(lib, kw, status):
    assert _rn(**kw) == status
    assert _lib.last_error() != ""


def test_rmsnorm_no_rows_and_atomic_mode_need_nothing(lib):
    assert _rn(M=0, x=0, w=0, dy=0, dx=0, dw=0, ws=0, ws_bytes=0) == _lib.GDR_OK


# gdr_validate_cu_seqlens: every invalid argument returns before any launch
@pytest.mark.parametrize("kw,status", [
    (dict(cu=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(res=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(n=0), _lib.GDR_ERR_INVALID_ARG),
    (dict(n=8193), _lib.GDR_ERR_INVALID_ARG),       # beyond the packed-batch maximum
    (dict(t=-1), _lib.GDR_ERR_INVALID_ARG),
    (dict(cu=FAKE + 2), _lib.GDR_ERR_INVALID_ARG),  # misaligned
    (dict(res=FAKE + 1), _lib.GDR_ERR_INVALID_ARG),
])
def test_validate_cu_seqlens_invalid_arguments(lib, kw, status):
    a = dict(cu=FAKE, n=4, t=100, res=FAKE)
    a.update(kw)
    assert _lib.gdr_validate_cu_seqlens(a["cu"], a["n"], a["t"], a["res"], 0, check=False) == status
    assert _lib.last_error() != ""
