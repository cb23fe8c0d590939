"""Races and determinism of the HIP kernels (GPU).

Delay injection: libgdr_delay.so is the same library compiled with
GDR_DEBUG_DELAY (include/libgdr_debug.h): after a pseudo-random subset of the
workgroup barriers of every kernel, chosen waves sleep.  A sleep changes no
arithmetic, so if every LDS hand-off between waves is ordered by a barrier,
that build's outputs with delays are bitwise equal to its outputs without.
The method (delay one side of a suspected race so its window opens, keep the
arithmetic, compare bitwise) is the one the review of FastVideo PR #1819
("[kernel] sm_100a CUDA backward for VSA block-sparse attention (blk64)")
uses to confirm a cross-warp race; the same review's second check, many
undelayed back-to-back runs compared bitwise, is the last test here.
"""
import os

import numpy as np
import pytest
import torch

from chunked_gated_delta_02_amd import _lib
from chunked_gated_delta_02_amd import inputs as gin
from chunked_gated_delta_02_amd import ops
from tests.gdr_cases import rel, run_gpu, say

pytestmark = pytest.mark.gpu

C = gin.CONFIGS

# every kernel and every template variant the workloads reach: fp32 and bf16
# paths, packed sequences, CP summaries and hand-off, 16/32/64-column scan
# tiles (the 8-wave output scan), wide values, snapshots saved or recomputed
RACE_CASES = {
    "fp32_tiny": (C[0], True),
    "bf16_varlen": (C[2].replace(name="race_varlen", H=4, lengths=[70, 0, 1, 200, 129, 64], len_range=None), True),
    "bf16_cp4_f16state": (C[3].replace(name="race_cp4", T=1000, H=2, cp_segments=4, h_store="f16"), True),
    "bf16_widev": (C[4].replace(name="race_widev", B=2, T=200, H=2), True),
    "bf16_recompute": (C[1].replace(name="race_recompute", B=2, T=333, H=3, has_h0=True), False),
    # 256 (sequence, head) units: the scans take their 32- and 64-column tiles
    "bf16_wide_tiles": (C[1].replace(name="race_wide_tiles", B=4, T=130, H=64), True),
}

# (wave, mod, iters): one wave lagging after every / every third barrier,
# and every wave lagging after a random half of its barriers
DELAYS = [(0, 1, 2), (3, 1, 2), (4, 1, 2), (7, 1, 2), (1, 3, 3), (-1, 2, 2)]


@pytest.fixture(scope="module")
def delay_lib():
    if not os.path.exists(_lib.DELAY_LIB_PATH):
        pytest.fail("libgdr_delay.so is not built (build() builds it beside libgdr.so)")
    with _lib.using(_lib.DELAY_LIB_PATH) as lib:
        _lib.gdr_debug_set_delay(-1, 1, 0)
        yield lib
        _lib.gdr_debug_set_delay(-1, 1, 0)


@pytest.mark.parametrize("case", sorted(RACE_CASES))
def test_delayed_waves_leave_results_bitwise_unchanged(case, delay_lib):
    w, saved = RACE_CASES[case]
    inp = gin.generate(w)
    say("[case] race %s: undelayed" % case)
    _lib.gdr_debug_set_delay(-1, 1, 0)
    base = run_gpu(w, inp, saved=saved)
    for i, (wave, mod, iters) in enumerate(DELAYS):
        say("[case] race %s: delay wave %d mod %d iters %d" % (case, wave, mod, iters))
        _lib.gdr_debug_set_delay(wave, mod, iters, salt=17 * i + 1)
        got = run_gpu(w, inp, saved=saved)
        for name in base:
            np.testing.assert_array_equal(got[name], base[name], err_msg="%s %s delay %s" % (
                case, name, (wave, mod, iters)))
    _lib.gdr_debug_set_delay(-1, 1, 0)


def test_delays_take_effect(delay_lib):
    # every wave sleeping ~16 x 8k cycles after every barrier: the serial scan
    # of a 16-chunk sequence alone passes 2 barriers per chunk, so the
    # delayed forward must take milliseconds longer than the undelayed one
    import time
    w = C[1].replace(name="race_timing", B=1, T=1024, H=2)
    inp = gin.generate(w)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}

    def fwd_time():
        torch.cuda.synchronize()
        t = time.perf_counter()
        ops.chunk_gdr_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], layout=w.layout, output_final_state=True)
        torch.cuda.synchronize()
        return time.perf_counter() - t

    _lib.gdr_debug_set_delay(-1, 1, 0)
    fwd_time()
    t0 = min(fwd_time() for _ in range(3))
    _lib.gdr_debug_set_delay(-1, 1, 16)
    t1 = min(fwd_time() for _ in range(3))
    _lib.gdr_debug_set_delay(-1, 1, 0)
    say("[race] forward %.3f ms undelayed, %.3f ms delayed" % (1e3 * t0, 1e3 * t1))
    assert t1 > t0 + 1e-3


def test_race_build_computes_what_the_production_build_does(delay_lib):
    # the instrumented build is the same computation (guards against testing
    # a build that differs in more than its barriers)
    w, saved = RACE_CASES["bf16_varlen"]
    inp = gin.generate(w)
    _lib.gdr_debug_set_delay(-1, 1, 0)
    a = run_gpu(w, inp, saved=saved)
    with _lib.using(_lib.LIB_PATH):
        b = run_gpu(w, inp, saved=saved)
    for name in a:
        assert rel(a[name], b[name]) <= 1e-6, name


def test_1000_back_to_back_runs_bitwise_identical():
    w = C[2].replace(name="repeat_varlen", H=4, lengths=[70, 0, 1, 200, 129, 64], len_range=None)
    say("[case] 1000 back-to-back runs %s" % w.name)
    inp = gin.generate(w)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}

    def once():
        o, hT, hs = ops.chunk_gdr_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], cu_seqlens=d["cu_seqlens"],
                                      h0=d["h0"], layout=w.layout, output_final_state=True)
        r = ops.chunk_gdr_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["do"], cu_seqlens=d["cu_seqlens"],
                              h0=d["h0"], dhT=d["dhT"], h_saved=hs, layout=w.layout)
        return [x for x in [o, hT] + [r[n] for n in sorted(r)] if x is not None]

    with _lib.using(_lib.LIB_PATH):   # the production build
        ref = once()
        assert len(ref) == 8
        bad = torch.zeros((), dtype=torch.int64, device="cuda")
        for _ in range(999):
            for x, y in zip(once(), ref):
                bad += (x != y).sum()
        torch.cuda.synchronize()
    assert int(bad) == 0


def test_full_size_runs_bitwise_identical():
    # the fixed-length workload at its full size, where every compute unit
    # runs a scan workgroup: repeated forward + backward calls must agree bit
    # for bit.  A race that corrupts a few hundred of 16.7 M elements stays
    # far inside a normwise tolerance, so only a bitwise repeat shows it.
    w = C[1]
    say("[case] full-size repeats %s" % w.name)
    inp = gin.generate(w)
    with _lib.using(_lib.LIB_PATH):
        ref = run_gpu(w, inp)
        for rep in range(3):
            got = run_gpu(w, inp)
            for name in ref:
                if ref[name] is None:
                    continue
                diff = int(np.count_nonzero(got[name] != ref[name]))
                assert diff == 0, "%s: %d elements differ on repeat %d" % (name, diff, rep + 1)
