"""gdr_chunk_fwd_noalloc, the forward for callers that cannot allocate: its
workspace is the library's static device array.  Through the C ABI, its
outputs must equal those of gdr_chunk_fwd (same kernels, caller workspace)
bit for bit, on two calls in a row -- the second smaller, on the array the
first left behind -- and problems too large for the array are refused on
the host."""
import pytest
import torch

from chunked_gated_delta_02_amd import _lib
from chunked_gated_delta_02_amd import inputs as gin
from chunked_gated_delta_02_amd import ops
from tests.gdr_cases import say

pytestmark = pytest.mark.gpu

C = gin.CONFIGS


def _outputs(w, inp, noalloc):
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k, v, beta, g = (d[n] for n in ("q", "k", "v", "beta", "g"))
    cu, h0 = d["cu_seqlens"], d["h0"]
    p = ops.make_problem(q, v, cu, w.layout, None, w.h_store, w.cp_segments)
    assert _lib.gdr_check(p) == _lib.GDR_OK
    N, H, K, V = inp["N"], w.H, w.DK, w.DV
    sshape = (N, H, K, V) if w.layout == "KV" else (N, H, V, K)
    # outputs start as NaN so that an unwritten element cannot match
    o = torch.full_like(v, float("nan"))
    hT = torch.full(sshape, float("nan"), dtype=torch.float32, device=dev)
    hs_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.h_store]
    hs = torch.full((_lib.gdr_h_saved_bytes(p) // hs_dt.itemsize,), float("nan"), dtype=hs_dt, device=dev)
    P = lambda t: 0 if t is None else t.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    say("[noalloc] %s %s: fwd workspace %d bytes" % (w.name, "static" if noalloc else "caller",
                                                     _lib.gdr_fwd_workspace_bytes(p)))
    if noalloc:
        _lib.gdr_chunk_fwd_noalloc(p, P(q), P(k), P(v), P(beta), P(g), P(cu), P(h0), P(o), P(hT), P(hs), stream)
    else:
        nb = _lib.gdr_fwd_workspace_bytes(p)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        _lib.gdr_chunk_fwd(p, P(q), P(k), P(v), P(beta), P(g), P(cu), P(h0), P(o), P(hT), P(hs), P(ws), nb,
                           stream)
    torch.cuda.synchronize()
    return o, hT, hs


def _same(a, b, what):
    # bit patterns: the NaN fill of elements neither call writes (chunk slots
    # past the last chunk of a packed batch in h_saved) compares equal too
    for x, y, name in zip(a, b, ("o", "hT", "h_saved")):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), \
            "%s: %s differs from gdr_chunk_fwd" % (what, name)
    assert not torch.isnan(a[0]).any() and not torch.isnan(a[1]).any(), "%s: o or hT not written" % what


def test_noalloc_forward_equals_caller_workspace_forward_twice():
    # a packed batch with context parallelism (every workspace region in use),
    # then a smaller fixed-length batch on the same static array
    big = C[2].replace(name="noalloc_varlen_cp2", H=4, lengths=[700, 0, 1, 333, 1500], len_range=None,
                       cp_segments=2)
    small = C[1].replace(name="noalloc_small", B=1, T=200, H=2, has_h0=True)
    for w in (big, small):
        inp = gin.generate(w)
        ref = _outputs(w, inp, noalloc=False)
        got = _outputs(w, inp, noalloc=True)
        _same(got, ref, w.name)


def test_noalloc_refuses_problems_beyond_its_array():
    # B = 2, T = 4096, H = 16, D = 128 needs ~200 MB of forward workspace:
    # refused on the host, nothing launched (the outputs stay untouched)
    dev = torch.device("cuda:0")
    q = torch.zeros(2, 4096, 16, 128, dtype=torch.bfloat16, device=dev)
    beta = torch.zeros(2, 4096, 16, dtype=torch.float32, device=dev)
    o = torch.full_like(q, 7.0)
    p = ops.make_problem(q, q, None, "KV", None, "f32", 1)
    assert _lib.gdr_fwd_workspace_bytes(p) > _lib.GDR_NOALLOC_SCRATCH_BYTES
    st = _lib.gdr_chunk_fwd_noalloc(p, q.data_ptr(), q.data_ptr(), q.data_ptr(), beta.data_ptr(),
                                    beta.data_ptr(), 0, 0, o.data_ptr(), 0, 0, 0, check=False)
    assert st == _lib.GDR_ERR_UNSUPPORTED
    assert "static workspace" in _lib.last_error()
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
