"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws random numbers and applies the input transforms of
the workload recipes (per-token L2 normalisation of k, sigmoid for beta,
log-sigmoid for g).  It holds none of the method's arithmetic and is the only
code shared by the tests, the benchmark and the oracle harness.

Recipe (all draws from ``torch.Generator('cpu').manual_seed(seed)``, in fp32,
in this order, then cast):
  [sequence lengths, varlen only]  q, k, v, beta-logits, g-logits, h0, dO, dh_T
  q, k, v ~ N(0, 1); k <- k / ||k||_2 per token; beta = sigmoid(N(0, 1));
  g = logsigmoid(N(g_mean, 1)); h0 ~ 0.1 N(0, 1); dO, dh_T ~ N(0, 1).
A draw whose tensor is not used by a workload is still made, so every tensor
of a workload depends only on (seed, shapes), not on which options are on.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    DK: int
    DV: int
    io_dtype: str = "bf16"          # "bf16" or "f32": q, k, v, o, dO and dq, dk, dv
    layout: str = "KV"              # state layout of h0, h_T, dh_T, dh0
    lengths: Optional[List[int]] = None  # varlen: sequence lengths (packed, B == 1)
    len_range: Optional[tuple] = None    # varlen: draw lengths uniformly in [lo, hi]
    n_seqs: int = 0                      # varlen: number of sequences to draw
    has_h0: bool = False
    has_hT: bool = True
    has_dhT: bool = True
    g_mean: float = 0.0
    h_store: str = "f32"            # dtype of the per-chunk state snapshots
    cp_segments: int = 1            # intra-card context-parallel segments
    seed: int = 0

    @property
    def varlen(self) -> bool:
        return self.lengths is not None or self.len_range is not None

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny fp32; fixed-length bf16 (the headline shape);
# varlen; long context with intra-card context parallelism; wide values.
CONFIGS = {
    0: Workload("tiny_fp32_T256_H2_D64", B=1, T=256, H=2, DK=64, DV=64, io_dtype="f32",
                layout="VK", has_h0=True, has_hT=True, has_dhT=True, seed=0),
    1: Workload("fixed_bf16_B2_T4096_H16_D128", B=2, T=4096, H=16, DK=128, DV=128,
                layout="KV", has_h0=False, has_hT=True, has_dhT=True, seed=1),
    2: Workload("varlen_bf16_N8_512-8192_H32_D128", B=1, T=0, H=32, DK=128, DV=128,
                layout="VK", len_range=(512, 8192), n_seqs=8, has_h0=True, has_hT=True,
                has_dhT=True, seed=2),
    3: Workload("longctx_bf16_T65536_H8_D128_cp8", B=1, T=65536, H=8, DK=128, DV=128,
                layout="KV", has_h0=False, has_hT=True, has_dhT=True, g_mean=3.0,
                cp_segments=8, seed=3),
    4: Workload("widev_bf16_B4_T8192_H32_DK128_DV256", B=4, T=8192, H=32, DK=128, DV=256,
                layout="KV", has_h0=True, has_hT=True, has_dhT=True, seed=4),
}

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def draw_lengths(w: Workload, gen: torch.Generator) -> List[int]:
    lo, hi = w.len_range
    return [int(x) for x in torch.randint(lo, hi + 1, (w.n_seqs,), generator=gen)]


def generate(w: Workload, device="cpu") -> dict:
    """Draw every tensor of workload `w`.

    Returns a dict with q, k, v, beta, g, do (token-major [B, T, H, D]),
    h0 / dhT (fp32 states in w.layout, or None), cu_seqlens (int32 or None),
    lengths, and N (number of sequences)."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    lengths = None
    if w.varlen:
        lengths = list(w.lengths) if w.lengths is not None else draw_lengths(w, gen)
        B, T = 1, int(sum(lengths))
        N = len(lengths)
    else:
        B, T, N = w.B, w.T, w.B
    H, DK, DV = w.H, w.DK, w.DV
    q = torch.randn(B, T, H, DK, generator=gen)
    k = torch.randn(B, T, H, DK, generator=gen)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    v = torch.randn(B, T, H, DV, generator=gen)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen))
    g = torch.nn.functional.logsigmoid(torch.randn(B, T, H, generator=gen) + w.g_mean)
    sshape = (N, H, DK, DV) if w.layout == "KV" else (N, H, DV, DK)
    h0 = 0.1 * torch.randn(*sshape, generator=gen)
    do = torch.randn(B, T, H, DV, generator=gen)
    dhT = torch.randn(*sshape, generator=gen)
    dt = _DT[w.io_dtype]
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), beta=beta.float(), g=g.float(),
               do=do.to(dt), h0=h0 if w.has_h0 else None, dhT=dhT if w.has_dhT else None,
               cu_seqlens=None, lengths=lengths, N=N)
    if lengths is not None:
        cu = [0]
        for L in lengths:
            cu.append(cu[-1] + L)
        out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
    if device != "cpu":
        for key in ("q", "k", "v", "beta", "g", "do", "h0", "dhT", "cu_seqlens"):
            if out[key] is not None:
                out[key] = out[key].to(device)
    return out


# ---------------------------------------------------------------------------
# RMSNorm backward inputs (the M x N bf16 sweep of the quack PR #101 page,
# "Rmsnorm backward fusing sum": M from 4k to 65k rows, N from 256 to 8k):
# x ~ N(0, 1) and dy ~ N(0, 1) in the io dtype, w = 1 + 0.1 N(0, 1) fp32,
# drawn in that order from torch.Generator('cpu').manual_seed(seed).

def generate_rmsnorm(M: int, N: int, io_dtype: str = "bf16", seed: int = 0) -> dict:
    gen = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(M, N, generator=gen)
    w = 1.0 + 0.1 * torch.randn(N, generator=gen)
    dy = torch.randn(M, N, generator=gen)
    dt = _DT[io_dtype]
    return dict(x=x.to(dt), w=w.float(), dy=dy.to(dt))
