#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule (forward + backward) on one
MI355X, through libgdr's C ABI.

One step = gdr_chunk_fwd (saving the per-chunk state snapshots) followed by
gdr_chunk_bwd on one batch of the fixed-length bf16 workload B=2, T=4096,
H=16, DK=DV=128 (seeded synthetic inputs, resident in HBM before the timed
region; between timed steps, outside the timed intervals, a 512 MiB write
evicts the Infinity Cache).  Prints ONE JSON line.  Per-kernel durations come
from a second pass of the same steps, in which libgdr records HIP events
around each launch on the call's stream (opt-in diagnostic timers); the
step time comes from the first pass, without those markers.  The dominant kernel's roofline uses its algorithmic
bytes (operator inputs read and outputs written once) and GEMM flops; the
per-kernel "kernels" entries use an implementation byte model (every tensor
and workspace buffer the kernel touches, once).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_FP32_FLOPS = 157.3e12    # MI355X fp32 matrix
PEAK_HBM = 8.0e12             # MI355X HBM3E bytes/s
CH = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("gdr", "rmsnorm_bwd"), default="gdr",
                    help="gdr: the gated delta rule step (default); rmsnorm_bwd: the fused RMSNorm "
                         "backward sweep with its three dw reduction modes")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the MFMA / bandwidth microbenchmarks (box-measured peaks)")
    ap.add_argument("--h-store", choices=("f32", "f16", "bf16"), default=None,
                    help="snapshot dtype (default: the workload's)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="between timed steps, write this many MiB to evict the 256 MB Infinity Cache "
                         "(outside the timed intervals; 0 = no flush)")
    ap.add_argument("--cp-segments", type=int, default=None,
                    help="intra-card context-parallel segments per sequence (default: the workload's)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step recorded into a HIP graph and replayed (ms_per_step_graph)")
    ap.add_argument("--recompute", action="store_true",
                    help="the forward keeps no state snapshots and the backward recomputes them "
                         "(default: the forward saves them for the backward)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed region, run one elementwise copy kernel of this many MiB "
                         "(fp32, read once + written once) as the scale reference of --pmc byte counters")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                         "WRITE_SIZE) of a run with --calibrate-copy-mib into profiles/<kernel>_<workload>_pmc.json")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# FLOP formula of the chunked algorithm (per token per head; 2mnk per GEMM,
# C^3/3 for the triangular inverse, elementwise work not counted)

def flops_fwd(K, V, C=CH):
    return 6 * K * V + 6 * C * K + 4 * C * V + C * C / 3.0


def flops_bwd(K, V, C=CH):
    return 14 * K * V + 18 * C * K + 10 * C * V + 13 * C * C / 3.0


# Algorithmic work of each kernel for one call: bytes of every tensor the
# kernel reads or writes, counted once, and the flops of the GEMMs it
# performs (2mnk), for NC chunk-heads, NP (sequence, head) pairs and NT
# token-heads.  e = io element size, hs = snapshot element size.

def kernel_model(name, mode, NC, NP, NT, K, V, e, hs, cp=1, C=CH):
    G = C * 4 * 3  # gate block per chunk-head: gamma, e^gamma, e^{gamma_L - gamma}
    if name in ("cp_scan_fwd", "cp_scan_bwd"):
        # segment summaries: the scan over all but one segment of every
        # sequence with DK + DV columns, no per-chunk outputs; writes the
        # DK x (DK + DV) summary per (segment, sequence, head)
        f = (cp - 1) / cp
        if name == "cp_scan_fwd":
            rd = f * NC * (2 * C * K * e + C * V * 4 + 4)
        else:
            rd = f * NC * (2 * C * K * e + C * V * 4 + K * V * 4 + 4)
        fl = f * NC * 4 * C * K * (K + V)
        return rd + (cp - 1) * NP * K * (K + V) * 4, fl
    if name in ("cp_chain_fwd", "cp_chain_bwd"):
        return (cp - 1) * NP * (K * (K + V) + K * V) * 4, (cp - 1) * NP * 2 * K * K * V
    if name == "wy":
        # reads q, k, v, beta, g (+ dO); writes the gate block, W, U (fp32)
        # and (fwd) K^T, Q, P (split: hi + lo) or (bwd) T, W^T, K,
        # scale P^T dO and scale (e^gamma Q)^T dO (fp32)
        fl = NC * (2 * C * C * K + C ** 3 / 3.0 + 2 * C * C * K + 2 * C * C * V + 2 * C * C * K)
        if mode == "fwd":
            rd = NT * (2 * K * e + V * e + 8)
            wr = NC * (G + C * K * e + C * V * 4 + K * C * e + C * K * e + C * C * e * (1 if e == 4 else 2))
        else:
            rd = NT * (2 * K * e + 2 * V * e + 8)
            wr = NC * (G + C * K * e + C * V * 4 + C * C * 4 + K * C * e + C * K * e + C * V * 4 + K * V * 4)
            fl += NC * (2 * C * C * V + 2 * C * K * V)
        return rd + wr, fl
    if name == "scan_fwd":
        # reads W, K^T, U (+ Q, P with the output); writes the snapshots
        # (+ o); h0 / hT per (sequence, head)
        rd = NC * (2 * C * K * e + C * V * 4 + 4) + NP * K * V * 4
        wr = NC * K * V * hs + NP * K * V * 4
        fl = NC * 4 * C * K * V
        if mode == "fwd":
            rd += NC * (C * K * e + C * C * e * (1 if e == 4 else 2))
            wr += NT * V * e
            fl += NC * (2 * C * K * V + 2 * C * C * V)
        return rd + wr, fl
    if name == "scan_bwd":
        # reads K, W^T, scale P^T dO and scale Qg^T dO (fp32); writes the dh
        # snapshots and dDelta (fp32); dhT / dh0 per (sequence, head)
        rd = NC * (2 * C * K * e + C * V * 4 + K * V * 4 + 4) + NP * K * V * 4
        wr = NC * (K * V * e + C * V * 4) + NP * K * V * 4
        return rd + wr, NC * 4 * C * K * V
    if name == "grad":
        # reads q, k, v, dO, beta, the gate block, T, W, U, the h and dh
        # snapshots and dDelta; writes dq, dk, dv, dbeta, dg
        rd = NT * (2 * K * e + 2 * V * e + 4) + NC * (G + C * C * 4 + C * K * e + C * V * 4
                                                      + K * V * hs + K * V * e + C * V * 4)
        wr = NT * (2 * K * e + V * e + 8)
        fl = NC * (8 * C * K * V + 6 * C * C * V + 14 * C * C * K + 4 * C ** 3)
        return rd + wr, fl
    if name == "plan":
        return 0, 0
    raise KeyError(name)


# Algorithmic bytes of a kernel: the operator's own inputs it must read and
# outputs it must write, each once (workspace and snapshots are implementation
# choices and are not counted).  k_grad reads every per-token input of the
# backward and writes every per-token gradient: per token-head
# (2 K e + 2 V e + 8) + (2 K e + V e + 8) bytes.  `states` = number of
# per-(sequence, head) fp32 state tensors the kernel reads or writes.

def algorithmic_bytes(name, mode, NT, NP, K, V, e, states):
    st = states * NP * K * V * 4
    if name == "grad":
        return NT * ((2 * K * e + 2 * V * e + 8) + (2 * K * e + V * e + 8))
    if name == "wy":
        return NT * (2 * K * e + V * e + 8 + (V * e if mode == "bwd" else 0))
    if name == "scan_fwd":
        return (NT * V * e if mode == "fwd" else 0) + st
    if name == "scan_bwd":
        return st
    return 0


# ---------------------------------------------------------------------------
class Hip:
    """Minimal HIP runtime access for events (ctypes on libamdhip64)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return e.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            # an event that was never recorded (kernel not launched): clear
            # the runtime's sticky error so later HIP calls do not report it
            self.lib.hipGetLastError()
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def metric_name(w, B, T, H, K, V):
    """The metric string of the workload that ran: the headline workload's is
    "GDR fwd+bwd tokens/s & TFLOPS (% bf16 MFMA peak), B=2 T=4096 H=16 D=128"."""
    dims = "D=%d" % K if K == V else "DK=%d DV=%d" % (K, V)
    if w.varlen:
        shape = "N=%d varlen T=%d H=%d %s" % (w.n_seqs or len(w.lengths or []), T, H, dims)
    else:
        shape = "B=%d T=%d H=%d %s" % (B, T, H, dims)
    extra = ""
    if w.cp_segments > 1:
        extra += " cp=%d" % w.cp_segments
    if w.h_store != "f32":
        extra += " h_store=%s" % w.h_store
    prec = "bf16" if w.io_dtype == "bf16" else "fp32"
    return "GDR fwd+bwd tokens/s & TFLOPS (%% %s MFMA peak), %s%s" % (prec, shape, extra)


def direction_bytes(mode, NT, NP, K, V, e, n_states):
    """Algorithmic HBM bytes of one direction: the operator's per-token
    inputs read and outputs written once, plus its per-(sequence, head) fp32
    states (h0 / h_T forward; h0, dh_T / dh0 backward)."""
    if mode == "fwd":
        per = 2 * K * e + 2 * V * e + 8
    else:
        per = (2 * K * e + 2 * V * e + 8) + (2 * K * e + V * e + 8)
    return NT * per + n_states * NP * K * V * 4


class Probe:
    """Box-measured ceilings from libgdr_probe.so: dense bf16 MFMA rate and
    streaming read / copy bandwidth, each timed with HIP events."""

    def __init__(self, hip, torch, dev, stream):
        path = os.path.join(ROOT, "chunked_gated_delta_02_amd", "libgdr_probe.so")
        if not os.path.exists(path):
            raise RuntimeError("%s is not built" % path)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.gdr_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
        L.gdr_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.gdr_probe_mfma_bf16_flops.restype = ctypes.c_double
        L.gdr_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        L.gdr_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_void_p]
        self.hip, self.torch, self.dev, self.stream = hip, torch, dev, stream

    def _time(self, fn, reps=5):
        a, b = self.hip.event(), self.hip.event()
        fn()
        best = None
        for _ in range(reps):
            self.hip.record(a, self.stream)
            rc = fn()
            self.hip.record(b, self.stream)
            if rc != 0:
                raise RuntimeError("probe launch failed: %d" % rc)
            self.torch.cuda.synchronize()
            ms = self.hip.elapsed_ms(a, b)
            best = ms if best is None else min(best, ms)
        self.hip.destroy(a)
        self.hip.destroy(b)
        return best

    def measure(self):
        torch = self.torch
        blocks, iters = 256 * 8, 4096
        out = torch.empty(blocks * 256, dtype=torch.float32, device=self.dev)
        rates = {}
        for shape in (16, 32):
            ms = self._time(lambda: self.lib.gdr_probe_mfma_bf16(shape, blocks, iters, out.data_ptr(),
                                                                 out.numel(), self.stream))
            rates[shape] = self.lib.gdr_probe_mfma_bf16_flops(shape, blocks, iters) / (ms * 1e-3)
        mfma = max(rates.values())
        nbytes = 2 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=self.dev)
        dst = torch.empty_like(src)
        rb = 256 * 16
        part = torch.empty(rb * 256, dtype=torch.float32, device=self.dev)
        ms_r = self._time(lambda: self.lib.gdr_probe_read(src.data_ptr(), nbytes, rb, part.data_ptr(),
                                                          part.numel(), self.stream))
        ms_c = self._time(lambda: self.lib.gdr_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, rb,
                                                          self.stream))
        del src, dst, part, out
        return {"bf16_mfma_tflops": round(mfma / 1e12, 1),
                "bf16_mfma_tflops_16x16x32": round(rates[16] / 1e12, 1),
                "bf16_mfma_tflops_32x32x16": round(rates[32] / 1e12, 1),
                "hbm_read_GBps": round(nbytes / (ms_r * 1e-3) / 1e9, 1),
                "hbm_copy_GBps": round(2 * nbytes / (ms_c * 1e-3) / 1e9, 1),
                "method": "libgdr_probe.so: %d workgroups x 4 waves x %d rounds of 8 independent "
                          "v_mfma_f32_16x16x32_bf16 or 4 of v_mfma_f32_32x32x16_bf16 (the faster "
                          "counts); 2 GiB streaming read and copy with 16-byte "
                          "accesses (copy counts read + write); best of 5 launches, HIP events"
                          % (blocks, iters)}


# the translation unit the counted kernel (k_grad) is compiled from
GRAD_SOURCES = ("chunked_gated_delta_02_amd/csrc/gdr_bwd.hip", "chunked_gated_delta_02_amd/csrc/gdr_kernels.h",
                "chunked_gated_delta_02_amd/csrc/gdr_device.h", "include/libgdr.h")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in GRAD_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def ingest_pmc(fetch_csv, write_csv, workload, copy_mib, dispatches_per_step):
    """Per-launch HBM bytes of k_grad from two rocprofv3 --pmc runs, scaled by
    what the same counters read for the calibration copy kernel."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if "MulFunctor" in k]
    copy_w = [v for k, v in write.items() if "MulFunctor" in k]
    if not copy_f or not copy_w:
        raise SystemExit("calibration copy kernel not found in the counter files")
    ref_kib = copy_mib * 1024.0
    f_scale = ref_kib / statistics.median(copy_f[0])
    w_scale = ref_kib / statistics.median(copy_w[0])
    name = [k for k in fetch if "k_grad" in k]
    if not name:
        raise SystemExit("k_grad not found in the counter files")
    kf = statistics.median(fetch[name[0]]) * f_scale * 1024.0
    kw = statistics.median(write[[k for k in write if "k_grad" in k][0]]) * w_scale * 1024.0
    out = {"kernel": "k_grad", "workload": workload, "source_hash": kernel_source_hash(),
           "fetch_bytes_per_launch": kf, "write_bytes_per_launch": kw,
           "hbm_bytes_per_launch": kf + kw,
           "calibration": {"copy_mib": copy_mib, "fetch_scale": f_scale, "write_scale": w_scale},
           "files": [os.path.basename(fetch_csv), os.path.basename(write_csv)]}
    path = os.path.join(ROOT, "profiles", "grad_bwd_%s_pmc.json" % workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
def cpu_baseline(w, inp, target_s):
    """The oracle (fp64, OpenMP over (sequence, head)) on a bounded sample of
    the workload: all sequences, a subset of heads sized to ~target_s."""
    import numpy as np
    from oracle import oracle
    threads = oracle.max_threads()
    H = w.H

    split = [0.0, 0.0]   # oracle seconds in the forward and backward calls

    def run(nh):
        sel = lambda t: t[:, :, :nh].double().numpy()
        q, k, v, beta, g, do = (sel(inp[n]) for n in ("q", "k", "v", "beta", "g", "do"))
        dhT = None if inp["dhT"] is None else inp["dhT"][:, :nh].double().numpy()
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, beta, g, layout=w.layout)
        t1 = time.perf_counter()
        oracle.bwd(q, k, v, beta, g, do, dhT=dhT, layout=w.layout)
        t2 = time.perf_counter()
        split[0], split[1] = t1 - t0, t2 - t1
        return t2 - t0

    # calibrate with as many heads as threads can take in one wave of pairs,
    # then grow the head subset (and, if the whole workload is quicker than
    # the target, repeat it) until the sample holds ~target_s of CPU work
    nh = max(1, min(H, threads // max(1, w.B)))
    t = run(nh)
    pairs_per_s = nh * w.B / t
    want = int(pairs_per_s * target_s / w.B)
    nh2 = max(1, min(H, want))
    reps = 1
    if nh2 > nh:
        nh, t = nh2, run(nh2)
    tf, tb = split
    if nh == H and t < target_s / 2:
        reps = max(1, int(target_s / t))
        t, tf, tb = 0.0, 0.0, 0.0
        for _ in range(reps):
            t += run(nh)
            tf += split[0]
            tb += split[1]
    tokens = reps * w.B * w.T * nh / H
    return {"value": tokens / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "fwd_tokens_per_s": tokens / tf, "bwd_tokens_per_s": tokens / tb,
            "sample": "fp64 oracle forward+backward on %d of %d heads of all %d sequences "
                      "(%d tokens x %d heads), %d repetition(s), %.1f s wall (forward %.1f s, "
                      "backward %.1f s, timed separately); tokens/s counts full tokens (all heads)"
                      % (nh, H, w.B, w.B * w.T, nh, reps, t, tf, tb)}


# The M x N points of the bf16 sweep on the quack PR #101 page ("Rmsnorm
# backward fusing sum"): M 4k..65k rows, N 256..8k.
RMSNORM_SWEEP = [(m, n) for n in (256, 512, 1024, 2048, 4096) for m in (4096, 8192, 16384, 32768, 65536)] + \
    [(m, 8192) for m in (4096, 16384, 65536)]


def bench_rmsnorm(args):
    """Fused RMSNorm backward: every sweep point in the three dw reduction
    modes, timed with HIP events (median of the timed launches, Infinity
    Cache flushed between launches), as a fraction of HBM bandwidth; the cost
    of determinism is the fixed-order time over the atomic one."""
    import torch
    from chunked_gated_delta_02_amd import _lib, rmsnorm
    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    hip = Hip()
    # inputs of the largest point, drawn on the device (seeded); smaller
    # points use leading slices
    gen = torch.Generator(device=dev).manual_seed(0)
    mmax = max(m for m, _ in RMSNORM_SWEEP)
    nmax = max(n for _, n in RMSNORM_SWEEP)
    xs = torch.randn(mmax * nmax, generator=gen, device=dev).to(torch.bfloat16)
    dys = torch.randn(mmax * nmax, generator=gen, device=dev).to(torch.bfloat16)
    w = 1.0 + 0.1 * torch.randn(nmax, generator=gen, device=dev)
    rstd = torch.rand(mmax, generator=gen, device=dev) + 0.5
    flush = torch.empty(args.flush_mib * (1 << 18), dtype=torch.float32, device=dev) if args.flush_mib else None
    steps = args.steps
    points = []
    for M, N in RMSNORM_SWEEP:
        x = xs[:M * N].view(M, N)
        dy = dys[:M * N].view(M, N)
        dx = torch.empty_like(x)
        dw = torch.zeros(N, dtype=torch.float32, device=dev)
        row = {"M": M, "N": N}
        for mode in ("fixed", "atomic", "separate"):
            mcode = rmsnorm.MODES[mode]
            ws = rmsnorm.workspace(M, N, mode, dev)
            nb = 0 if ws is None else ws.numel()
            P = lambda t: 0 if t is None else t.data_ptr()

            def call():
                _lib.gdr_rmsnorm_bwd(M, N, _lib.GDR_BF16, P(x), P(w[:N]), P(dy), P(rstd[:M]), 1e-6, P(dx),
                                     P(dw), mcode, P(ws), nb, stream)

            for _ in range(args.warmup):
                call()
            evs = [(hip.event(), hip.event()) for _ in range(steps)]
            for a_, b_ in evs:
                if flush is not None:
                    flush.fill_(1.0)
                hip.record(a_, stream)
                call()
                hip.record(b_, stream)
            torch.cuda.synchronize()
            ts = sorted(hip.elapsed_ms(a_, b_) for a_, b_ in evs)
            for a_, b_ in evs:
                hip.destroy(a_)
                hip.destroy(b_)
            row[mode + "_us"] = round(1e3 * ts[len(ts) // 2], 2)
        byt = 3 * M * N * 2 + N * 4 * 2 + M * 4      # x, dy read, dx written (bf16); w, dw; rstd
        row["algorithmic_bytes"] = byt
        row["fixed_GBps"] = round(byt / (row["fixed_us"] * 1e-6) / 1e9, 1)
        row["fixed_frac_hbm"] = round(byt / (row["fixed_us"] * 1e-6) / PEAK_HBM, 4)
        row["determinism_cost"] = round(row["fixed_us"] / row["atomic_us"], 3)
        row["fused_speedup_vs_separate"] = round(row["separate_us"] / row["fixed_us"], 3)
        points.append(row)
    import math
    gm = lambda xs_: math.exp(sum(math.log(v) for v in xs_) / len(xs_))
    big = max(points, key=lambda r: r["algorithmic_bytes"])
    res = {"metric": "fused RMSNorm backward (bf16) time per call in three dw reduction modes",
           "workload": "rmsnorm_bwd_bf16_sweep_M4096-65536_N256-8192",
           "unit": "us", "steps": steps, "warmup": args.warmup, "cache_flush_mib": args.flush_mib,
           "points": points,
           "summary": {"geomean_determinism_cost_fixed_over_atomic": round(gm([r["determinism_cost"] for r in points]), 3),
                       "geomean_fused_speedup_fixed_vs_separate": round(gm([r["fused_speedup_vs_separate"] for r in points]), 3),
                       "largest_point": {"M": big["M"], "N": big["N"], "fixed_us": big["fixed_us"],
                                         "fixed_frac_hbm": big["fixed_frac_hbm"]}},
           "roofline": {"bound": "hbm", "achieved": big["fixed_GBps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": big["fixed_frac_hbm"], "kernel": "k_rmsnorm_bwd (fixed-order mode)",
                        "traffic": None}}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.workload == "rmsnorm_bwd":
        if args.gpus != 1:
            print("bench.py runs on one GPU only (asked for --gpus %d)" % args.gpus, file=sys.stderr)
            sys.exit(2)
        bench_rmsnorm(args)
        return
    if args.ingest_pmc:
        from chunked_gated_delta_02_amd import inputs as gin
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], gin.CONFIGS[args.config].name,
                   args.calibrate_copy_mib or 256, 1)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(asked for --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from chunked_gated_delta_02_amd import _lib, inputs as gin, ops

    w = gin.CONFIGS[args.config]
    if args.h_store:
        w = w.replace(h_store=args.h_store)
    if args.cp_segments:
        w = w.replace(cp_segments=args.cp_segments)
    inp = gin.generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k, v, beta, g, do = (d[n] for n in ("q", "k", "v", "beta", "g", "do"))
    h0, dhT, cu = d["h0"], d["dhT"], d["cu_seqlens"]
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = inp["N"]
    p = ops.make_problem(q, v, cu, w.layout, None, w.h_store, w.cp_segments)
    st = _lib.gdr_check(p)
    if st != _lib.GDR_OK:
        raise _lib.GDRError(st, _lib.last_error())
    sshape = (N, H, K, V) if w.layout == "KV" else (N, H, V, K)
    o = torch.empty_like(v)
    hT = torch.empty(sshape, dtype=torch.float32, device=dev)
    hs_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.h_store]
    h_saved = None if args.recompute else \
        torch.empty(_lib.gdr_h_saved_bytes(p) // hs_dt.itemsize, dtype=hs_dt, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbeta, dg = torch.empty_like(beta), torch.empty_like(g)
    dh0 = torch.empty(sshape, dtype=torch.float32, device=dev)
    fws = _lib.gdr_fwd_workspace_bytes(p)
    bws = _lib.gdr_bwd_workspace_bytes(p, h_saved is not None)
    wsf = torch.empty(fws, dtype=torch.uint8, device=dev)
    wsb = torch.empty(bws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = lambda t: 0 if t is None else t.data_ptr()

    def fwd(st=None):
        _lib.gdr_chunk_fwd(p, P(q), P(k), P(v), P(beta), P(g), P(cu), P(h0), P(o), P(hT), P(h_saved),
                           P(wsf), fws, stream if st is None else st)

    def bwd(st=None):
        _lib.gdr_chunk_bwd(p, P(q), P(k), P(v), P(beta), P(g), P(cu), P(h0), P(h_saved), P(do), P(dhT),
                           P(dq), P(dk), P(dv), P(dbeta), P(dg), P(dh0), P(wsb), bws, stream if st is None else st)

    hip = Hip()
    nk = len(_lib.KERNELS)
    # warm-up steps are the timed steps without the timing: the same cache
    # flush and step events around the same calls, so that the first timed
    # step pays no first-use cost of the flush buffer or of recording events
    # (measured: with bare fwd/bwd warm-up steps the host lagged the GPU in
    # the first timed pass and its steps read 10-25 us longer)
    flush = torch.empty(args.flush_mib * (1 << 18), dtype=torch.float32, device=dev) if args.flush_mib else None
    wev = [(hip.event(), hip.event(), hip.event()) for _ in range(args.warmup)]
    for s in range(args.warmup):
        if flush is not None:
            flush.fill_(float(s))
        hip.record(wev[s][0], stream)
        fwd()
        hip.record(wev[s][1], stream)
        bwd()
        hip.record(wev[s][2], stream)
    torch.cuda.synchronize()

    # timed region: K steps, each bracketed by its own events.  Between steps
    # (outside the brackets) a write of flush_mib MiB evicts the Infinity
    # Cache, so no step starts with its inputs cached from the previous one.
    # A second pass of K steps, after the timed one, has libgdr record
    # per-kernel events around each launch (the breakdown and the roofline);
    # those markers add small gaps, so the step time comes from the first.
    evs = [[[hip.event() for _ in range(2 * nk)] for _ in range(2)] for _ in range(args.steps)]
    # per step: start, end of forward (= start of backward), end
    sev = [(hip.event(), hip.event(), hip.event()) for _ in range(args.steps)]
    sevb = [(hip.event(), hip.event(), hip.event()) for _ in range(args.steps)]
    sev2 = [(hip.event(), hip.event()) for _ in range(args.steps)]

    def timed_pass(evl):
        for s in range(args.steps):
            if flush is not None:
                flush.fill_(float(s))
            hip.record(evl[s][0], stream)
            fwd()
            hip.record(evl[s][1], stream)
            bwd()
            hip.record(evl[s][2], stream)

    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    timed_pass(sev)          # pass A: the K timed steps of the result
    torch.cuda.synchronize()
    t_host1 = time.perf_counter()
    for s in range(args.steps):
        if flush is not None:
            flush.fill_(float(s))
        hip.record(sev2[s][0], stream)
        _lib.gdr_set_kernel_timers(evs[s][0])
        fwd()
        _lib.gdr_set_kernel_timers(evs[s][1])
        bwd()
        hip.record(sev2[s][1], stream)
    _lib.gdr_set_kernel_timers(None)
    timed_pass(sevb)         # pass B: the same steps again, after the marker pass
    torch.cuda.synchronize()

    def split_ms(evl):
        return ([hip.elapsed_ms(a, c) for a, _, c in evl], [hip.elapsed_ms(a, b) for a, b, _ in evl],
                [hip.elapsed_ms(b, c) for _, b, c in evl])

    stepA, fwdA, bwdA = split_ms(sev)
    stepB, fwdB, bwdB = split_ms(sevb)
    ms_step = sum(stepA) / args.steps
    ms_step_timed = sum(hip.elapsed_ms(a, b) for a, b in sev2) / args.steps
    med = lambda xs: sorted(xs)[len(xs) // 2] if len(xs) % 2 else 0.5 * sum(sorted(xs)[len(xs) // 2 - 1:len(xs) // 2 + 1])
    if args.calibrate_copy_mib:
        # scale reference for --pmc byte counters: fp32 elementwise multiply by
        # one, reading and writing calibrate_copy_mib MiB once each
        src = torch.ones(args.calibrate_copy_mib * (1 << 18), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # per-kernel averages
    per = {}
    for phase_i, phase in enumerate(("fwd", "bwd")):
        for ki, kname in enumerate(_lib.KERNELS):
            times = []
            for s in range(args.steps):
                a, b = evs[s][phase_i][2 * ki], evs[s][phase_i][2 * ki + 1]
                try:
                    times.append(hip.elapsed_ms(a, b))
                except RuntimeError:
                    break  # kernel not launched in this phase
            if len(times) == args.steps:
                per["%s.%s" % (phase, kname)] = sum(times) / len(times)
    for row in evs:
        for ph in row:
            for e in ph:
                hip.destroy(e)
    for evl in (sev, sevb, sev2):
        for tup in evl:
            for e_ in tup:
                hip.destroy(e_)
    graph_ms = None
    if args.graph:
        # the same step recorded once into a HIP graph (the library issues
        # only kernel launches) and replayed, flushed and timed like pass A
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream(dev).cuda_stream
            fwd(cs)
            bwd(cs)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            gr.replay()
        sevg = [(hip.event(), hip.event()) for _ in range(args.steps)]
        for s in range(args.steps):
            if flush is not None:
                flush.fill_(float(s))
            hip.record(sevg[s][0], stream)
            gr.replay()
            hip.record(sevg[s][1], stream)
        torch.cuda.synchronize()
        graph_ms = [hip.elapsed_ms(a, b) for a, b in sevg]
        for tup in sevg:
            for e_ in tup:
                hip.destroy(e_)
        del gr
    del flush
    peaks = None
    if not args.no_probe:
        peaks = Probe(hip, torch, dev, stream).measure()

    tokens = B * T
    NT = B * T * H
    if cu is None:
        NC = B * ((T + CH - 1) // CH) * H
    else:
        lens = (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1]).tolist()
        NC = sum((n + CH - 1) // CH for n in lens) * H
    NP = N * H
    e = q.element_size()
    hs = hs_dt.itemsize
    fl_f = NT * flops_fwd(K, V)
    fl_b = NT * flops_bwd(K, V)
    peak = PEAK_BF16_FLOPS if q.dtype == torch.bfloat16 else PEAK_FP32_FLOPS

    kernels = {}
    for key, ms in per.items():
        phase, kname = key.split(".")
        byt, fl = kernel_model(kname, phase, NC, NP, NT, K, V, e, hs, w.cp_segments)
        kernels[key] = {"avg_us": round(ms * 1e3, 2), "GBps": round(byt / (ms * 1e-3) / 1e9, 1),
                        "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2)}
    dom = max(per, key=per.get)
    phase, kname = dom.split(".")
    _, fl = kernel_model(kname, phase, NC, NP, NT, K, V, e, hs, w.cp_segments)
    nstates = {("scan_fwd", "fwd"): (h0 is not None) + 1, ("scan_bwd", "bwd"): (dhT is not None) + 1}
    byt = algorithmic_bytes(kname, phase, NT, NP, K, V, e, nstates.get((kname, phase), 0))
    t_dom = per[dom] * 1e-3
    if byt / PEAK_HBM >= fl / peak:
        roof = {"bound": "hbm", "achieved": round(byt / t_dom / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(byt / t_dom / PEAK_HBM, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(fl / t_dom / 1e12, 2), "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": round(fl / t_dom / peak, 4)}
    roof["kernel"] = "k_%s (%s)" % (kname, phase)
    roof["avg_us"] = round(per[dom] * 1e3, 2)
    roof["algorithmic_bytes"] = int(byt)
    roof["algorithmic_flops"] = int(fl)
    roof["traffic"] = measured_traffic(kname + "_" + phase, w.name)

    fwd_ms = med(fwdA + fwdB)
    bwd_ms = med(bwdA + bwdB)
    nst_f = (h0 is not None) + 1                     # h0 read, h_T written
    nst_b = (h0 is not None) + (dhT is not None) + 1  # h0, dh_T read, dh0 written
    directions = {}
    for mode, ms, fl_, ns in (("fwd", fwd_ms, fl_f, nst_f), ("bwd", bwd_ms, fl_b, nst_b)):
        byt_d = direction_bytes(mode, NT, NP, K, V, e, ns)
        directions[mode] = {
            "median_ms": round(ms, 4),
            "tflops": round(fl_ / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(fl_ / (ms * 1e-3) / peak, 4),
            "algorithmic_bytes": int(byt_d),
            "algorithmic_GBps": round(byt_d / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(byt_d / (ms * 1e-3) / PEAK_HBM, 4),
            "kernels_sum_ms": round(sum(v for k2, v in per.items() if k2.startswith(mode + ".")), 4)}
        if peaks:
            directions[mode]["frac_measured_mfma"] = round(fl_ / (ms * 1e-3) / (peaks["bf16_mfma_tflops"] * 1e12), 4)
            directions[mode]["frac_measured_hbm"] = round(byt_d / (ms * 1e-3) / (peaks["hbm_read_GBps"] * 1e9), 4)
    res = {
        "metric": metric_name(w, B, T, H, K, V),
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "DK": K, "DV": V, "chunk": CH,
                   "layout": w.layout, "h_store": w.h_store, "cp_segments": w.cp_segments, "seed": w.seed,
                   "snapshots": "recomputed" if args.recompute else "saved",
                   "parallelism": "single GPU"},
        "tflops": {"fwd+bwd": round((fl_f + fl_b) / (ms_step * 1e-3) / 1e12, 2),
                   "fwd_kernels": round(fl_f / (fwd_ms * 1e-3) / 1e12, 2) if fwd_ms else None,
                   "bwd_kernels": round(fl_b / (bwd_ms * 1e-3) / 1e12, 2) if bwd_ms else None},
        "frac_bf16_peak": round((fl_f + fl_b) / (ms_step * 1e-3) / PEAK_BF16_FLOPS, 4),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "directions": directions,
        "protocol": {"warmup_steps": args.warmup, "timed_steps_per_pass": args.steps, "passes": 2,
                     "value_from": "mean of pass A",
                     "median_ms_per_step": round(med(stepA + stepB), 4),
                     "pass_median_ms_per_step": [round(med(stepA), 4), round(med(stepB), 4)],
                     "between_passes": "the per-kernel marker pass",
                     "cache_flush_mib": args.flush_mib},
        "host_wall_ms_per_step": round((t_host1 - t_host0) * 1e3 / args.steps, 4),
        "ms_per_step_with_kernel_timers": round(ms_step_timed, 4),
        "cache_flush_mib": args.flush_mib,
        "kernels": kernels,
        "roofline": roof,
        "peaks_measured": peaks,
        "cpu_baseline": None,
    }
    if graph_ms is not None:
        res["ms_per_step_graph"] = round(med(graph_ms), 4)
        res["graph_note"] = ("the same step recorded into one HIP graph and replayed; median of %d replays, "
                             "flushed like pass A (value stays the eager pass)" % len(graph_ms))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
