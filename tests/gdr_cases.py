"""Shared helpers of the GPU parity tests: run libgdr (through its C ABI) and
the fp64 oracle on the same seeded inputs and compare every output."""
from __future__ import annotations

import sys

import numpy as np
import torch

from chunked_gated_delta_02_amd import inputs as gin
from chunked_gated_delta_02_amd import ops
from oracle import oracle

TOL = {"f32": 1e-5, "bf16": 5e-3}
OUTS_FWD = ("o", "hT")
OUTS_BWD = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(x, y) -> float:
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    n = np.linalg.norm(y)
    d = np.linalg.norm(x - y)
    return float(d / n) if n > 0 else float(d)


def to64(t):
    return None if t is None else t.detach().to("cpu").double().numpy()


def run_gpu(w: gin.Workload, inp: dict, h_store=None, saved=True, device="cuda", cp_fwd=None, cp_bwd=None):
    """libgdr forward + backward; returns dict of fp64 NumPy arrays.  The
    context-parallel segment counts default to the workload's."""
    dev = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    hs = h_store or w.h_store
    cp_fwd = w.cp_segments if cp_fwd is None else cp_fwd
    cp_bwd = w.cp_segments if cp_bwd is None else cp_bwd
    say("[gpu] %s fwd: B=%d T=%d H=%d DK=%d DV=%d io=%s layout=%s h0=%s varlen=%s h_store=%s cp=%d/%d" % (
        w.name, dev["q"].shape[0], dev["q"].shape[1], w.H, w.DK, w.DV, w.io_dtype, w.layout,
        inp["h0"] is not None, inp["cu_seqlens"] is not None, hs, cp_fwd, cp_bwd))
    o, hT, h_saved = ops.chunk_gdr_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"],
                                       cu_seqlens=dev["cu_seqlens"], h0=dev["h0"], layout=w.layout,
                                       output_final_state=True, save_states=saved, h_store=hs,
                                       cp_segments=cp_fwd)
    torch.cuda.synchronize()
    say("[gpu] %s bwd (saved states: %s)" % (w.name, saved))
    r = ops.chunk_gdr_bwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["do"],
                          cu_seqlens=dev["cu_seqlens"], h0=dev["h0"], dhT=dev["dhT"],
                          h_saved=h_saved, layout=w.layout, h_store=hs, cp_segments=cp_bwd)
    torch.cuda.synchronize()
    out = dict(o=to64(o), hT=to64(hT))
    out.update({k: to64(v) for k, v in r.items()})
    return out


def run_oracle(w: gin.Workload, inp: dict, heads=None):
    """fp64 oracle on the same values (optionally a subset of heads)."""
    sel = (lambda t: t) if heads is None else (lambda t: None if t is None else t[:, :, heads])
    ssel = (lambda t: t) if heads is None else (lambda t: None if t is None else t[:, heads])
    q, k, v, beta, g, do = (sel(to64(inp[n])) for n in ("q", "k", "v", "beta", "g", "do"))
    h0, dhT = ssel(to64(inp["h0"])), ssel(to64(inp["dhT"]))
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    say("[oracle] %s heads=%s" % (w.name, "all" if heads is None else list(heads)))
    o, hT = oracle.fwd(q, k, v, beta, g, cu_seqlens=cu, h0=h0, layout=w.layout)
    r = oracle.bwd(q, k, v, beta, g, do, cu_seqlens=cu, h0=h0, dhT=dhT, layout=w.layout)
    out = dict(o=o, hT=hT)
    out.update(r)
    return out


def compare(w: gin.Workload, got: dict, ref: dict, heads=None, tol=None):
    tol = tol if tol is not None else TOL[w.io_dtype]
    errs = {}
    for name in OUTS_FWD + OUTS_BWD:
        x = got[name]
        if heads is not None:
            x = x[:, heads] if name in ("hT", "dh0") else x[:, :, heads]
        errs[name] = rel(x, ref[name])
    say("[errors] %s: %s" % (w.name, " ".join("%s=%.2e" % kv for kv in errs.items())))
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, "normwise error above %.0e: %s" % (tol, bad)
    return errs
