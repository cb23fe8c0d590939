"""libgdr for MI355X: the chunked gated delta rule (forward and fused
backward) as hand-written gfx950 HIP kernels behind a C ABI
(``include/libgdr.h``), with a thin PyTorch binding.

    from chunked_gated_delta_02_amd import chunk_gdr
    o, hT = chunk_gdr(q, k, v, beta, g, h0=None, layout="KV")

The HIP library is loaded on first use; if it has not been built the call
raises (there is no CPU or PyTorch fallback).
"""
from .ops import (ChunkGDRFunction, chunk_gdr, chunk_gdr_bwd, chunk_gdr_fwd, make_problem,  # noqa: F401
                  validate_cu_seqlens)
from ._lib import GDRError  # noqa: F401

__all__ = ["chunk_gdr", "chunk_gdr_fwd", "chunk_gdr_bwd", "ChunkGDRFunction", "make_problem", "GDRError",
           "validate_cu_seqlens"]
