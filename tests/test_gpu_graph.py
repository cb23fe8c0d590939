"""HIP-graph capture of libgdr calls.  The library never allocates,
synchronises or clears memory with a memset, so a caller can record its
launches into a graph: here the forward and backward (and the
allocation-free forward, and the fused RMSNorm backward in its fixed-order
mode) are called through the C ABI under ``torch.cuda.graph`` capture, with
every buffer allocated before the capture.  Each graph is replayed three
times with eager work and a synchronisation between the replays (the
outputs refilled with NaN first), and every replay must equal the eager
call bit for bit."""
import pytest
import torch

from chunked_gated_delta_02_amd import _lib, rmsnorm
from chunked_gated_delta_02_amd import inputs as gin
from chunked_gated_delta_02_amd import ops
from tests.gdr_cases import say

pytestmark = pytest.mark.gpu

C = gin.CONFIGS
DEV = torch.device("cuda:0")
P = lambda t: 0 if t is None else t.data_ptr()   # noqa: E731

CASES = {
    "fixed_ragged": C[1].replace(name="graph_fixed", B=2, T=333, H=3),
    "varlen_cp2": C[2].replace(name="graph_varlen_cp2", H=4, lengths=[70, 0, 1, 200, 129, 64], len_range=None,
                               cp_segments=2),
    "fp32_vk_h0": C[0].replace(name="graph_fp32", B=2, T=150, H=2, has_h0=True),
}


class _Problem:
    """Every buffer of one forward + backward, allocated up front."""

    def __init__(self, w):
        inp = gin.generate(w)
        d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        self.d, self.w = d, w
        q, v = d["q"], d["v"]
        self.p = ops.make_problem(q, v, d["cu_seqlens"], w.layout, None, w.h_store, w.cp_segments)
        assert _lib.gdr_check(self.p) == _lib.GDR_OK
        N, H, K, V = inp["N"], w.H, w.DK, w.DV
        sshape = (N, H, K, V) if w.layout == "KV" else (N, H, V, K)
        hs_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.h_store]
        self.out = dict(
            o=torch.empty_like(v), hT=torch.empty(sshape, dtype=torch.float32, device=DEV),
            hs=torch.empty(max(_lib.gdr_h_saved_bytes(self.p), 16) // hs_dt.itemsize, dtype=hs_dt, device=DEV),
            dq=torch.empty_like(q), dk=torch.empty_like(d["k"]), dv=torch.empty_like(v),
            dbeta=torch.empty_like(d["beta"]), dg=torch.empty_like(d["g"]),
            dh0=torch.empty(sshape, dtype=torch.float32, device=DEV))
        self.fb = _lib.gdr_fwd_workspace_bytes(self.p)
        self.bb = _lib.gdr_bwd_workspace_bytes(self.p, True)
        self.fws = torch.empty(max(self.fb, 1), dtype=torch.uint8, device=DEV)
        self.bws = torch.empty(max(self.bb, 1), dtype=torch.uint8, device=DEV)

    def poison(self):
        for t in self.out.values():
            t.view(torch.uint8).fill_(0xFF)   # NaN in every float type

    def call(self, noalloc=False):
        d, o, p = self.d, self.out, self.p
        stream = torch.cuda.current_stream(DEV).cuda_stream
        if noalloc:
            _lib.gdr_chunk_fwd_noalloc(p, P(d["q"]), P(d["k"]), P(d["v"]), P(d["beta"]), P(d["g"]),
                                       P(d["cu_seqlens"]), P(d["h0"]), P(o["o"]), P(o["hT"]), P(o["hs"]), stream)
        else:
            _lib.gdr_chunk_fwd(p, P(d["q"]), P(d["k"]), P(d["v"]), P(d["beta"]), P(d["g"]), P(d["cu_seqlens"]),
                               P(d["h0"]), P(o["o"]), P(o["hT"]), P(o["hs"]), P(self.fws), self.fb, stream)
        _lib.gdr_chunk_bwd(p, P(d["q"]), P(d["k"]), P(d["v"]), P(d["beta"]), P(d["g"]), P(d["cu_seqlens"]),
                           P(d["h0"]), P(o["hs"]), P(d["do"]), P(d["dhT"]), P(o["dq"]), P(o["dk"]), P(o["dv"]),
                           P(o["dbeta"]), P(o["dg"]), P(o["dh0"]), P(self.bws), self.bb, stream)

    def snapshot(self):
        # o, h_T and every gradient (not the opaque snapshot buffer, whose
        # slots past the last chunk of a packed batch are never written)
        return {k: v.clone() for k, v in self.out.items() if k != "hs"}


def _replay_and_compare(g, prob, ref, what):
    for rep in range(3):
        prob.poison()
        torch.randn(1 << 20, device=DEV).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(prob.out[k].view(torch.uint8), v.view(torch.uint8)), \
                "%s: replay %d differs from the eager call in %s" % (what, rep, k)


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("noalloc", [False, True])
def test_forward_backward_graph_replays_equal_eager(case, noalloc):
    w = CASES[case]
    prob = _Problem(w)
    say("[graph] %s noalloc=%s: eager reference" % (w.name, noalloc))
    prob.poison()
    prob.call(noalloc)          # eager (also sets up the static workspace's address once)
    torch.cuda.synchronize()
    ref = prob.snapshot()
    for k, v in ref.items():
        assert not torch.isnan(v.float()).any(), "%s: eager %s not written" % (w.name, k)
    g = torch.cuda.CUDAGraph()
    say("[graph] %s: capture" % w.name)
    with torch.cuda.graph(g):
        prob.call(noalloc)
    _replay_and_compare(g, prob, ref, w.name)


def test_rmsnorm_fixed_mode_graph_replays_equal_eager():
    # dw is accumulated into, so the graph clears it first with a fill kernel
    # (a memset node is avoided); the arrival counters return to zero at the
    # end of every call, so each replay starts from a clean workspace
    M, N = 3000, 2048
    inp = gin.generate_rmsnorm(M, N, "bf16", seed=5)
    x, dy, w = (inp[n].to(DEV) for n in ("x", "dy", "w"))
    dx = torch.empty_like(x)
    dw = torch.empty(N, dtype=torch.float32, device=DEV)
    ws = rmsnorm.workspace(M, N, "fixed", DEV)
    nb = ws.numel()

    def call():
        dw.zero_()
        _lib.gdr_rmsnorm_bwd(M, N, _lib.GDR_BF16, P(x), P(w), P(dy), 0, 1e-6, P(dx), P(dw),
                             _lib.GDR_REDUCE_FIXED, P(ws), nb, torch.cuda.current_stream(DEV).cuda_stream)

    call()
    torch.cuda.synchronize()
    ref = (dx.clone(), dw.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        dx.view(torch.uint8).fill_(0xFF)
        dw.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), ref[0].view(torch.int16)), "replay %d: dx" % rep
        assert torch.equal(dw.view(torch.int32), ref[1].view(torch.int32)), "replay %d: dw" % rep
        assert int(ws[:512].count_nonzero()) == 0, "replay %d: counters not back at zero" % rep
