/* libgdr_probe.h -- measurement probes (libgdr_probe.so), not part of the
 * gated delta rule library.  They measure the two ceilings the operator's
 * kernels are reported against -- dense bf16 MFMA throughput and HBM
 * streaming bandwidth -- on the GPU at hand, so that the roofline fractions
 * can be stated against measured as well as vendor peaks.
 *
 * Pointers are device pointers; every call launches one kernel on `stream`
 * (a hipStream_t, NULL = the null stream) and returns a hipError_t value
 * (0 = hipSuccess).  Arguments are checked on the host before the launch:
 * invalid ones return hipErrorInvalidValue and launch nothing.  The caller
 * times the launch (HIP events) and owns every buffer.
 */
#ifndef LIBGDR_PROBE_H
#define LIBGDR_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `blocks` workgroups of 256 threads each run `iters` rounds of independent
 * bf16 MFMA chains per wave: shape 16 = 8 chains of v_mfma_f32_16x16x32_bf16,
 * shape 32 = 4 chains of v_mfma_f32_32x32x16_bf16.  One float per thread is
 * written to out (out_elems >= 256 * blocks, else nothing is launched). */
int gdr_probe_mfma_bf16(int shape, int blocks, int iters, float* out, size_t out_elems, void* stream);
/* flops that gdr_probe_mfma_bf16(shape, blocks, iters, ...) executes */
double gdr_probe_mfma_bf16_flops(int shape, int blocks, int iters);

/* reads `bytes` (a multiple of 16, src 16-byte aligned) once with 16-byte
 * loads, grid-stride over `blocks` workgroups of 256 threads; one partial
 * sum per thread to out (out_elems >= 256 * blocks). */
int gdr_probe_read(const void* src, size_t bytes, int blocks, float* out, size_t out_elems, void* stream);

/* copies `bytes` (a multiple of 16, both pointers 16-byte aligned) from src
 * to dst with 16-byte loads and stores, grid-stride. */
int gdr_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDR_PROBE_H */
