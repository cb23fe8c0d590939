/*
 * libgdr.h -- C ABI of libgdr: the chunked gated delta rule (forward and fused
 * backward) on AMD Instinct MI355X (gfx950).
 *
 * The operator.  FlashQLA PR #34 ("SM120/121 : Add support for fused backward
 * kernel") names it in its "Summary" section: the chunked gated delta rule and
 * its fused backward fused_gdr_bwd.  Its "Current status" section lists the
 * feature set this header exposes: fixed-length and variable-length inputs,
 * KV/VK state layouts, initial and final states, autograd, and intra-card
 * context parallelism.  The draft of the same PR (page "[WIP] SM120 fused
 * backward kernel", first paragraph) stores the chunk state h in fp16.  The
 * pages print no formula; per (sequence, head) the library computes the
 * standard gated delta recurrence, state S in R^{DV x DK}:
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale S_t q_t,       S_0 = h0 (zeros if absent),  h_T = S_T
 *
 * in chunks of 64 tokens, and its exact gradient.
 *
 * Memory conventions (every pointer is a DEVICE pointer unless stated):
 *   q, k              [B, T, H, DK]   io dtype, contiguous, token-major
 *   v, o, dO          [B, T, H, DV]   io dtype
 *   beta, g           [B, T, H]       fp32; g is the natural-log decay
 *   cu_seqlens        int32 [N + 1], non-decreasing, cu[0] = 0, cu[N] <= T;
 *                     packed variable-length batch: B must be 1 and sequence
 *                     n occupies tokens [cu[n], cu[n+1])
 *   h0, hT, dhT, dh0  fp32, [N, H, DK, DV] (KV: h = S^T) or [N, H, DV, DK] (VK)
 *   dq, dk            [B, T, H, DK] io dtype;  dv [B, T, H, DV] io dtype
 *   dbeta, dg         [B, T, H] fp32
 * N is B for fixed-length batches and len(cu_seqlens) - 1 for packed ones.
 * All buffers must be 16-byte aligned.  Outputs may not alias inputs.
 *
 * Ownership and errors.  The caller owns and allocates every buffer,
 * including the workspace; the library never allocates, keeps no state
 * between calls (apart from the opt-in per-thread diagnostic timers below)
 * and is safe to call concurrently from several host threads on different
 * streams (each call needs its own workspace).  Every argument
 * error is detected on the host before any launch: the call returns a status,
 * launches nothing and writes nothing.  gdr_last_error() returns a message
 * for the calling thread's last failed call.  Work is enqueued on the given
 * HIP stream (NULL = default stream) and the call returns without
 * synchronising.  Contents of cu_seqlens are never read on the host; a
 * cu_seqlens that breaks the contract above gives unspecified results.
 * Results are bitwise reproducible for identical inputs (no floating-point
 * atomics).
 */
#ifndef LIBGDR_H
#define LIBGDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1, /* bad dimension, null required pointer, misalignment */
  GDR_ERR_UNSUPPORTED = 2, /* valid request outside what the library implements */
  GDR_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required    */
  GDR_ERR_HIP = 4          /* a HIP launch failed                                */
} gdr_status;

enum { GDR_F32 = 0, GDR_BF16 = 1, GDR_F16 = 2 };
enum { GDR_LAYOUT_KV = 0, GDR_LAYOUT_VK = 1 };

typedef struct {
  int32_t batch;         /* B (1 for packed batches)                               */
  int32_t seqlen;        /* T: tokens per sequence, or total packed tokens          */
  int32_t num_seqs;      /* N: must equal batch when varlen == 0                    */
  int32_t varlen;        /* 1: packed batch described by cu_seqlens                 */
  int32_t heads;         /* H >= 1                                                  */
  int32_t dk;            /* 64 or 128                                               */
  int32_t dv;            /* multiple of 64, 64..512                                 */
  int32_t chunk;         /* must be 64                                              */
  int32_t io_dtype;      /* GDR_F32 or GDR_BF16: q,k,v,o,dO,dq,dk,dv                */
  int32_t h_store_dtype; /* per-chunk state snapshots: GDR_F32, GDR_F16 or GDR_BF16
                            (GDR_F32 only when io_dtype is GDR_F32)                 */
  int32_t layout;        /* GDR_LAYOUT_KV or GDR_LAYOUT_VK for h0,hT,dhT,dh0       */
  int32_t cp_segments;   /* intra-card context parallelism: each sequence is cut
                            into this many chunk-aligned segments whose state
                            scans run concurrently (1 = off, at most 1024);
                            see below                                               */
  float scale;           /* <= 0 selects dk^-1/2                                    */
} gdr_problem;

/* Intra-card context parallelism (the "intra-card CP" of FlashQLA PR #34,
 * "Current status").  The state recursion of a chunk is affine in the state,
 * h' = M_c h + b_c with M_c = e^{gamma_L} I - Kt^T W, so a sequence cut into
 * segments is scanned in three steps: every segment but the last computes its
 * transition [prod M_c | state from zero] by scanning the augmented state
 * [I | 0] (the identity columns take no input); a short serial pass hands
 * the start state from segment to segment in fp32; then every segment runs
 * the ordinary scan from its start state.  The backward mirrors this on dh
 * with the transposed transitions.  Results equal cp_segments = 1 up to
 * rounding; the forward and the backward of one problem may use different
 * cp_segments (the saved snapshots do not depend on it). */

/* Validate a problem description.  Reads no tensor contents (the convention
 * the support check of FastVideo PR #1819 follows, section "Semantics"):
 * every decision is taken from the sizes, dtypes and flags alone. */
gdr_status gdr_check(const gdr_problem* p);

/* Workspace sizes in bytes (0 if the problem is invalid).  The backward
 * needs less when the caller passes the forward's saved states. */
size_t gdr_fwd_workspace_bytes(const gdr_problem* p);
size_t gdr_bwd_workspace_bytes(const gdr_problem* p, int have_h_saved);

/* Size of the per-chunk state snapshots that gdr_chunk_fwd can save for
 * gdr_chunk_bwd: one DV x DK state per chunk slot and head, in
 * h_store_dtype (an opaque buffer: only gdr_chunk_bwd reads it).  Chunk
 * slots: B * ceil(T/64) for fixed-length batches, ceil(T/64) + N for packed
 * ones. */
size_t gdr_h_saved_bytes(const gdr_problem* p);

/* Forward.  Writes o; writes hT if non-NULL; writes the state snapshots to
 * h_saved if non-NULL (for a later gdr_chunk_bwd); with h_saved NULL no
 * snapshot is written anywhere (a later backward recomputes them).  h0 may
 * be NULL (zeros).  cu_seqlens must be non-NULL exactly when p->varlen is
 * 1. */
gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, const int32_t* cu_seqlens,
                         const float* h0, void* o, float* hT, void* h_saved, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Backward: gradients of L with dL/do = dO and dL/dh_T = dhT (NULL = zero).
 * Writes each of dq, dk, dv, dbeta, dg and dh0 that is non-NULL (a NULL
 * gradient is not written; the others are unchanged by its absence).
 * h_saved: the snapshots written by gdr_chunk_fwd for the same inputs, or
 * NULL to recompute them. */
gdr_status gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, const int32_t* cu_seqlens,
                         const float* h0, const void* h_saved, const void* dO, const float* dhT,
                         void* dq, void* dk, void* dv, float* dbeta, float* dg, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the forward of
 * gdr_chunk_fwd with no workspace argument.  It runs the same kernels on a
 * static device array of the library, GDR_NOALLOC_SCRATCH_BYTES bytes on
 * every GPU it runs on (kept until the process ends), and allocates nothing.
 * Problems whose gdr_fwd_workspace_bytes() exceeds that size are refused
 * with GDR_ERR_UNSUPPORTED before any launch.  The array is shared by every
 * call on the same GPU: calls whose launches can overlap there (different
 * streams with no ordering between them) race; calls ordered on one stream
 * do not.  The stream must belong to the current device.  Arguments and
 * outputs as in gdr_chunk_fwd. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v,
                                 const float* beta, const float* g, const int32_t* cu_seqlens,
                                 const float* h0, void* o, float* hT, void* h_saved, void* stream);

/* Checks, on the device, the contract of a packed batch's cu_seqlens that
 * gdr_chunk_fwd / gdr_chunk_bwd assume without reading it on the host:
 * cu_seqlens[0] = 0 and every later entry in [previous entry, total_tokens].
 * One kernel is launched on `stream`; it writes to the device int *result
 * the smallest index i in [0, num_seqs] whose entry breaks the contract, or
 * -1 if none does (result needs no clearing beforehand; read it after the
 * stream has passed the launch).  The forward and backward themselves clamp
 * a broken cu_seqlens into range, so it cannot make them read or write out
 * of bounds, but their results are then unspecified; this check (which the
 * Python binding runs before each packed call when GDR_VALIDATE=1 is set in
 * the environment) says so explicitly.  Arguments: num_seqs in [1, 8192],
 * total_tokens >= 0, both pointers non-NULL and 4-byte aligned; otherwise an
 * error is returned and nothing is launched. */
gdr_status gdr_validate_cu_seqlens(const int32_t* cu_seqlens, int num_seqs, int total_tokens, int32_t* result,
                                   void* stream);

/* Diagnostics: per-kernel timing with caller-owned HIP events.
 * Kernel ids of the launches a forward / backward call makes: */
enum {
  GDR_KERNEL_PLAN = 0,       /* packed batches: cu_seqlens -> chunk table          */
  GDR_KERNEL_WY = 1,         /* gamma, T = (I + A)^-1, W, U, P (and bwd extras)    */
  GDR_KERNEL_SCAN_FWD = 2,   /* state scan with fused output (bwd: recompute only) */
  GDR_KERNEL_SCAN_BWD = 3,   /* reverse dh scan                                    */
  GDR_KERNEL_GRAD = 4,       /* fused chunk-parallel gradient kernel               */
  GDR_KERNEL_CP_SCAN_FWD = 5,  /* cp_segments > 1: segment transitions (forward)    */
  GDR_KERNEL_CP_CHAIN_FWD = 6, /* cp_segments > 1: start-state hand-off (forward)   */
  GDR_KERNEL_CP_SCAN_BWD = 7,  /* cp_segments > 1: segment transitions (backward)   */
  GDR_KERNEL_CP_CHAIN_BWD = 8, /* cp_segments > 1: dh hand-off (backward)           */
  GDR_NUM_KERNELS = 9
};
/* events: NULL to switch timing off for the calling thread, else an array of
 * 2 * GDR_NUM_KERNELS hipEvent_t handles (start, stop per kernel id; NULL
 * entries are skipped).  Later gdr_chunk_fwd / gdr_chunk_bwd calls on this
 * thread record start / stop on their stream immediately before / after each
 * launch of a timed kernel.  The array is copied; the events stay owned by
 * the caller.  Only the calling thread is affected. */
gdr_status gdr_set_kernel_timers(void* const* events);

const char* gdr_status_string(gdr_status s);
/* Message describing the calling thread's last failed call ("" if none). */
const char* gdr_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDR_H */
