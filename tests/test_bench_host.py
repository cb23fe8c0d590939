"""Host logic of bench.py (no GPU): the metric's FLOP formula, the roofline's
algorithmic bytes, the one-GPU contract and the PMC traffic bookkeeping."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_flop_formula_per_token_head():
    # 2mnk per GEMM of the chunked forward / backward and C^3/3 for the
    # triangular inverse, at DK = DV = 128, C = 64
    assert bench.flops_fwd(128, 128) == pytest.approx(6 * 128 * 128 + 6 * 64 * 128 + 4 * 64 * 128 + 64 * 64 / 3)
    assert round(bench.flops_fwd(128, 128)) == 181589
    assert round(bench.flops_bwd(128, 128)) == 476501


def test_gradient_kernel_algorithmic_bytes():
    # inputs q, k, v, dO (bf16) and beta, g read once; dq, dk, dv (bf16) and
    # dbeta, dg written once: 1808 bytes per token-head at DK = DV = 128
    nt = 2 * 4096 * 16
    assert bench.algorithmic_bytes("grad", "bwd", nt, 32, 128, 128, 2, 0) == nt * 1808 == 236978176


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_ingest_scales_by_the_copy_kernel_and_checks_the_sources(tmp_path, monkeypatch):
    # the copy kernel over 64 MiB reads back half of its bytes on FETCH_SIZE
    # and all of them on WRITE_SIZE: k_grad's counters are scaled the same way
    (tmp_path / "profiles").mkdir()
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    copy = "void at::native::MulFunctor<float>(...)"
    _counter_csv(fcsv, "FETCH_SIZE", [(copy, 32 * 1024), ("gdr::k_grad<...>", 1000.0), ("gdr::k_grad<...>", 1000.0)])
    _counter_csv(wcsv, "WRITE_SIZE", [(copy, 64 * 1024), ("gdr::k_grad<...>", 300.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "aaaa")
    bench.ingest_pmc(str(fcsv), str(wcsv), "wl", 64, 1)
    got = bench.measured_traffic("grad_bwd", "wl")
    assert got == pytest.approx(1000.0 * 2 * 1024 + 300.0 * 1024)
    # figures taken on other kernel sources are not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "bbbb")
    assert bench.measured_traffic("grad_bwd", "wl") is None


def test_metric_string_names_the_workload_that_ran():
    from chunked_gated_delta_02_amd import inputs as gin
    C = gin.CONFIGS
    assert bench.metric_name(C[1], 2, 4096, 16, 128, 128) == \
        "GDR fwd+bwd tokens/s & TFLOPS (% bf16 MFMA peak), B=2 T=4096 H=16 D=128"
    assert bench.metric_name(C[4], 4, 8192, 32, 128, 256).endswith("B=4 T=8192 H=32 DK=128 DV=256")
    assert bench.metric_name(C[3], 1, 65536, 8, 128, 128).endswith("B=1 T=65536 H=8 D=128 cp=8")
    assert "N=8 varlen" in bench.metric_name(C[2], 1, 34000, 32, 128, 128)
    assert "fp32 MFMA" in bench.metric_name(C[0], 1, 256, 2, 64, 64)
    assert bench.metric_name(C[1].replace(h_store="f16"), 2, 4096, 16, 128, 128).endswith("h_store=f16")


def test_direction_algorithmic_bytes():
    # forward: q, k, v, beta, g read and o written (2 K e + 2 V e + 8 per
    # token-head) plus h_T; backward: q, k, v, dO, beta, g read and dq, dk,
    # dv, dbeta, dg written, plus dh_T read and dh0 written
    nt, npairs = 2 * 4096 * 16, 32
    state = npairs * 128 * 128 * 4
    assert bench.direction_bytes("fwd", nt, npairs, 128, 128, 2, 1) == nt * (4 * 128 * 2 + 8) + state
    assert bench.direction_bytes("bwd", nt, npairs, 128, 128, 2, 2) == nt * 1808 + 2 * state
