/* gdr_rmsnorm.h -- fused RMSNorm backward of libgdr, with a selectable
 * reduction of the weight gradient.
 *
 * The operator is the RMSNorm backward whose per-workgroup weight-gradient
 * partials Dao-AILab/quack PR #101 ("Rmsnorm backward fusing sum",
 * description) reduces inside the backward kernel instead of in a separate
 * sum kernel; the review thread of the same page debates whether such an
 * in-kernel reduction must be deterministic.  Here the choice is the
 * caller's (gdr_reduce_mode), and the default is deterministic.
 *
 * Forward (not part of the library): per row x of length N,
 *   r = (mean_j x_j^2 + eps)^(-1/2),   y_j = w_j x_j r.
 * Backward, for a cotangent dy, with xhat = r x:
 *   dx_j = r (w_j dy_j - xhat_j mean_k(w_k dy_k xhat_k))
 *   dw_j += sum over rows of dy_j xhat_j
 *
 * All pointers are device pointers; work is launched on `stream` (a
 * hipStream_t) with no host synchronisation.  Errors in the arguments are
 * returned before any launch and nothing is written.
 */
#ifndef GDR_RMSNORM_H
#define GDR_RMSNORM_H

#include <stddef.h>

#include "libgdr.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  /* default: every workgroup writes its partial of dw to the workspace; the
   * last workgroup of each group of 32 to finish sums the group's partials
   * in workgroup order, and the last group to finish sums the group sums in
   * group order and adds them to dw -- all inside the one kernel, with
   * bitwise reproducible results */
  GDR_REDUCE_FIXED = 0,
  /* every workgroup adds its partial to dw with floating-point atomics: no
   * workspace, but the order of the additions (and so the rounding of dw)
   * varies from run to run */
  GDR_REDUCE_ATOMIC = 1,
  /* partials to the workspace, then a second kernel sums them in workgroup
   * order (deterministic; the unfused form the page compares against) */
  GDR_REDUCE_SEPARATE = 2
} gdr_reduce_mode;

/* Workspace bytes gdr_rmsnorm_bwd needs for (M, N, mode); 0 for GDR_REDUCE_ATOMIC
 * or an invalid request. */
size_t gdr_rmsnorm_bwd_workspace_bytes(int M, int N, int mode);

/* RMSNorm backward over M rows of N elements.
 *   x, dy : [M, N] in io_dtype (GDR_BF16 or GDR_F32), rows contiguous
 *   w     : [N] fp32
 *   rstd  : [M] fp32, the forward's r per row; NULL = computed from x and eps
 *   dx    : [M, N] in io_dtype (written)
 *   dw    : [N] fp32, ACCUMULATED: dw += sum_rows dy * xhat (zero it first
 *           for a plain gradient)
 * Limits: M >= 0, 8 <= N <= 8192, N a multiple of 8; x, dy, dx, w, dw and
 * the workspace 16-byte aligned.
 * Workspace (GDR_REDUCE_FIXED, GDR_REDUCE_SEPARATE): at least
 * gdr_rmsnorm_bwd_workspace_bytes(M, N, mode) bytes, caller-owned.  In
 * GDR_REDUCE_FIXED mode its first 512 bytes hold the workgroups' arrival
 * counters: they must be zero when the workspace is first used (allocate
 * it zeroed), and every call leaves them zero again.  Calls sharing one
 * workspace must be ordered (one stream). */
gdr_status gdr_rmsnorm_bwd(int M, int N, int io_dtype, const void* x, const float* w, const void* dy,
                           const float* rstd, float eps, void* dx, float* dw, int mode, void* workspace,
                           size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_RMSNORM_H */
