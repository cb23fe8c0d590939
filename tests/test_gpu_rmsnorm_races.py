"""Races in the fused RMSNorm backward (GPU), by delay injection.

libgdr_delay.so (the race-test build, include/libgdr_debug.h) lets chosen
waves sleep after the kernel's barriers and around the hand-offs of the
fixed-order weight-gradient reduction: before a workgroup stores its
partial, and in the last arriver of a group (and of the final level) before
it takes the acquire and reads the others' partials.  A sleep changes no
arithmetic, so if every hand-off is ordered -- the cross-wave row sums by
barriers, the cross-workgroup partials by the release / acquire of the
arrival counters -- the outputs with delays equal those without, bit for
bit, and the counters return to zero after every call.  The same method
serves the gated delta rule kernels in test_gpu_races.py."""
import os

import pytest
import torch

from chunked_gated_delta_02_amd import _lib, rmsnorm
from chunked_gated_delta_02_amd import inputs as gin
from tests.gdr_cases import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
P = lambda t: 0 if t is None else t.data_ptr()   # noqa: E731

# one shape per row layout: a wave per row (N <= 1024), the whole workgroup
# per row with a barrier per row sum (N = 2048, two workgroups per CU, 16
# groups of the two-level reduction), and the widest rows (8192)
SHAPES = [(5000, 512), (20000, 2048), (3000, 8192)]
DELAYS = [(0, 1, 2), (3, 1, 2), (1, 3, 3), (-1, 2, 2)]


@pytest.fixture(scope="module")
def delay_lib():
    if not os.path.exists(_lib.DELAY_LIB_PATH):
        pytest.fail("libgdr_delay.so is not built (build() builds it beside libgdr.so)")
    with _lib.using(_lib.DELAY_LIB_PATH) as lib:
        _lib.gdr_debug_set_delay(-1, 1, 0)
        yield lib
        _lib.gdr_debug_set_delay(-1, 1, 0)


def _run(M, N, mode, inp, ws):
    x, dy, w = (inp[n].to(DEV) for n in ("x", "dy", "w"))
    dx = torch.empty_like(x)
    dw = torch.zeros(N, dtype=torch.float32, device=DEV)
    nb = 0 if ws is None else ws.numel()
    _lib.gdr_rmsnorm_bwd(M, N, _lib.GDR_BF16, P(x), P(w), P(dy), 0, 1e-6, P(dx), P(dw), rmsnorm.MODES[mode],
                         P(ws), nb, torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    return dx, dw


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("mode", ["fixed", "separate"])
def test_delayed_waves_leave_rmsnorm_bitwise_unchanged(M, N, mode, delay_lib):
    inp = gin.generate_rmsnorm(M, N, "bf16", seed=11)
    ws = rmsnorm.workspace(M, N, mode, DEV)
    _lib.gdr_debug_set_delay(-1, 1, 0)
    dx0, dw0 = _run(M, N, mode, inp, ws)
    for i, (wave, mod, iters) in enumerate(DELAYS):
        say("[case] rmsnorm race %dx%d %s: delay wave %d mod %d iters %d" % (M, N, mode, wave, mod, iters))
        _lib.gdr_debug_set_delay(wave, mod, iters, salt=31 * i + 5)
        dx, dw = _run(M, N, mode, inp, ws)
        assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16)), (M, N, mode, wave, mod, iters)
        assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32)), (M, N, mode, wave, mod, iters)
        if mode == "fixed":
            assert int(ws[:512].count_nonzero()) == 0, "arrival counters not back at zero"
    _lib.gdr_debug_set_delay(-1, 1, 0)


def test_race_build_computes_what_the_production_build_does(delay_lib):
    M, N = 20000, 2048
    inp = gin.generate_rmsnorm(M, N, "bf16", seed=11)
    _lib.gdr_debug_set_delay(-1, 1, 0)
    a = _run(M, N, "fixed", inp, rmsnorm.workspace(M, N, "fixed", DEV))
    with _lib.using(_lib.LIB_PATH):
        b = _run(M, N, "fixed", inp, rmsnorm.workspace(M, N, "fixed", DEV))
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_rmsnorm_delays_take_effect(delay_lib):
    # every wave sleeping ~16 x 8k cycles at every delay point: with two
    # barriers per row (the whole workgroup shares each 2048-wide row) the
    # delayed call must take milliseconds longer
    import time
    M, N = 4000, 2048
    inp = gin.generate_rmsnorm(M, N, "bf16", seed=3)
    ws = rmsnorm.workspace(M, N, "fixed", DEV)

    def t_call():
        torch.cuda.synchronize()
        t = time.perf_counter()
        _run(M, N, "fixed", inp, ws)
        return time.perf_counter() - t

    _lib.gdr_debug_set_delay(-1, 1, 0)
    t_call()
    t0 = min(t_call() for _ in range(3))
    _lib.gdr_debug_set_delay(-1, 1, 16)
    t1 = min(t_call() for _ in range(3))
    _lib.gdr_debug_set_delay(-1, 1, 0)
    say("[race] rmsnorm %.3f ms undelayed, %.3f ms delayed" % (1e3 * t0, 1e3 * t1))
    assert t1 > t0 + 1e-3
