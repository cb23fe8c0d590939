"""GPU parity of the fused RMSNorm backward (include/gdr_rmsnorm.h) against
the fp64 oracle, in its three reduction modes.  dx is held to the normwise
bound of its io dtype (5e-3 bf16, 1e-5 fp32) and to element-wise bounds; dw
(fp32 sums over all rows) to 1e-5.  The fixed-order and separate modes must
be bitwise reproducible and the fixed-order mode must leave its arrival
counters at zero; the atomic mode is held to the tolerance only."""
import numpy as np
import pytest
import torch

from chunked_gated_delta_02_amd import _lib
from chunked_gated_delta_02_amd import inputs as gin
from chunked_gated_delta_02_amd import rmsnorm
from oracle import rmsnorm_oracle as ro
from tests.gdr_cases import rel, rel_emax, say

pytestmark = pytest.mark.gpu

TOL_DX = {"bf16": 5e-3, "f32": 1e-5}
EMAX_DX = {"bf16": 8e-3, "f32": 2e-5}
TOL_DW = 1e-5
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib_built():
    _lib.load()


def _run(M, N, io, mode, given_rstd=True, seed=0, dw0=None, ws=None):
    inp = gin.generate_rmsnorm(M, N, io, seed)
    r = ro.rstd(inp["x"], EPS).astype(np.float32)       # the forward's r, rounded to fp32
    dev = torch.device("cuda:0")
    x, w, dy = inp["x"].to(dev), inp["w"].to(dev), inp["dy"].to(dev)
    rs = torch.from_numpy(r).to(dev) if given_rstd else None
    dw = None if dw0 is None else dw0.clone().to(dev)
    say("[rmsnorm] M=%d N=%d io=%s mode=%s rstd=%s" % (M, N, io, mode, "given" if given_rstd else "recomputed"))
    dx, dwo = rmsnorm.rmsnorm_bwd(x, w, dy, rstd=rs, eps=EPS, dw=dw, mode=mode, ws=ws)
    torch.cuda.synchronize()
    return inp, r, dx, dwo


def _check(inp, r, dx, dw, io, given_rstd=True, dw0=None):
    rr = r.astype(np.float64) if given_rstd else None
    rdx, rdw = ro.backward(inp["x"], inp["w"], inp["dy"], r=rr, eps=EPS)
    if dw0 is not None:
        rdw = rdw + dw0.double().numpy()
    gdx = dx.double().cpu().numpy()
    gdw = dw.double().cpu().numpy()
    e = (rel(gdx, rdx), rel_emax(gdx, rdx), rel(gdw, rdw))
    say("[errors] dx=%.2e dx_emax=%.2e dw=%.2e" % e)
    assert e[0] <= TOL_DX[io] and e[1] <= EMAX_DX[io] and e[2] <= TOL_DW, e


SHAPES = [(1, 8), (3, 24), (1000, 256), (777, 1000), (513, 2048), (300, 3000), (200, 4104), (129, 8192)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("mode", ["fixed", "atomic", "separate"])
def test_parity_bf16(M, N, mode):
    inp, r, dx, dw = _run(M, N, "bf16", mode)
    _check(inp, r, dx, dw, "bf16")


@pytest.mark.parametrize("M,N", [(37, 64), (700, 1536), (90, 6000)])
@pytest.mark.parametrize("given", [True, False])
def test_parity_fp32_and_recomputed_rstd(M, N, given):
    inp, r, dx, dw = _run(M, N, "f32", "fixed", given_rstd=given)
    _check(inp, r, dx, dw, "f32", given_rstd=given)


def test_dw_is_accumulated_into():
    dw0 = torch.linspace(-1, 1, 512, dtype=torch.float32)
    for mode in ("fixed", "atomic", "separate"):
        inp, r, dx, dw = _run(600, 512, "bf16", mode, dw0=dw0)
        _check(inp, r, dx, dw, "bf16", dw0=dw0)


def test_fixed_and_separate_modes_are_bitwise_reproducible_and_counters_return_to_zero():
    M, N = 20000, 2048    # 512 workgroups: 16 first-level groups
    for mode in ("fixed", "separate"):
        ws = rmsnorm.workspace(M, N, mode, torch.device("cuda:0"))
        first = None
        for _ in range(4):
            _, _, dx, dw = _run(M, N, "bf16", mode, ws=ws)
            if first is None:
                first = (dx.clone(), dw.clone())
            else:
                assert torch.equal(dx.view(torch.int16), first[0].view(torch.int16))
                assert torch.equal(dw.view(torch.int32), first[1].view(torch.int32)), mode
            if mode == "fixed":
                assert int(ws[:512].count_nonzero()) == 0, "arrival counters not returned to zero"


def test_no_rows_leaves_dw_unchanged():
    dev = torch.device("cuda:0")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=dev)
    w = torch.ones(256, device=dev)
    dw0 = torch.full((256,), 3.0, device=dev)
    dx, dw = rmsnorm.rmsnorm_bwd(x, w, x.clone(), dw=dw0.clone())
    torch.cuda.synchronize()
    assert dx.numel() == 0 and torch.equal(dw, dw0)


def test_full_size_page_sweep_corner():
    # the largest point of the page's sweep, M = 65536, N = 8192: dx on
    # sampled rows (rows are independent), dw over every row (the oracle
    # summed block by block: dw is a sum over rows)
    M, N = 65536, 8192
    inp, r, dx, dw = _run(M, N, "bf16", "fixed", seed=3)
    rows = np.r_[0:3, 4097:4100, 40000:40003, M - 3:M]
    rdx, _ = ro.backward(inp["x"][rows], inp["w"], inp["dy"][rows], r=r[rows].astype(np.float64))
    gdx = dx[torch.from_numpy(rows).to(dx.device)].double().cpu().numpy()
    rdw = np.zeros(N)
    for b in range(0, M, 8192):
        rdw += ro.backward(inp["x"][b:b + 8192], inp["w"], inp["dy"][b:b + 8192],
                           r=r[b:b + 8192].astype(np.float64))[1]
    e = (rel(gdx, rdx), rel(dw.double().cpu().numpy(), rdw))
    say("[errors] full-size dx(sampled rows)=%.2e dw=%.2e" % e)
    assert e[0] <= TOL_DX["bf16"] and e[1] <= TOL_DW
