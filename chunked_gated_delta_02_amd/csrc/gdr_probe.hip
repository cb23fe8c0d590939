// gdr_probe.hip -- microbenchmarks that measure, on the GPU at hand, the two
// ceilings the gated delta rule kernels are compared against: dense bf16
// MFMA throughput and HBM streaming bandwidth.  Built into libgdr_probe.so
// (include/libgdr_probe.h), separate from libgdr; the benchmark times the
// launches with HIP events and reports the rates beside the vendor figures.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libgdr_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Every wave keeps PROBE_CHAINS independent accumulator chains of
// v_mfma_f32_16x16x32_bf16 in flight, enough to cover the instruction's
// dependent-issue latency, so the loop runs at the matrix units' issue rate.
#define PROBE_CHAINS 8

__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float* out) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((l + j) & 7));
    b[j] = (__bf16)(0.002f * (float)((l * 3 + j) & 7));
  }
  f32x4 c[PROBE_CHAINS];
#pragma unroll
  for (int i = 0; i < PROBE_CHAINS; ++i) c[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < PROBE_CHAINS; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PROBE_CHAINS; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// the same with v_mfma_f32_32x32x16_bf16 (16 accumulators per lane per chain)
__global__ __launch_bounds__(256) void k_probe_mfma32(int iters, float* out) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((l + j) & 7));
    b[j] = (__bf16)(0.002f * (float)((l * 3 + j) & 7));
  }
  f32x16 c[PROBE_CHAINS / 2];
#pragma unroll
  for (int i = 0; i < PROBE_CHAINS / 2; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < PROBE_CHAINS / 2; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PROBE_CHAINS / 2; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// streaming read: 16-byte loads, grid-stride; one partial sum per thread
__global__ __launch_bounds__(256) void k_probe_read(const f32x4* src, size_t n16, float* out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    acc += __builtin_nontemporal_load(src + i);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

// streaming copy: 16-byte loads and stores, grid-stride
__global__ __launch_bounds__(256) void k_probe_copy(const f32x4* src, f32x4* dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

int gdr_probe_mfma_bf16(int shape, int blocks, int iters, float* out, size_t out_elems, void* stream) {
  if ((shape != 16 && shape != 32) || blocks < 1 || iters < 1 || !out || (size_t)blocks * 256 > out_elems)
    return (int)hipErrorInvalidValue;
  if (shape == 16) hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else hipLaunchKernelGGL(k_probe_mfma32, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}

double gdr_probe_mfma_bf16_flops(int shape, int blocks, int iters) {
  // 4 waves per block; 16 x 16 x 32: PROBE_CHAINS instructions per round,
  // 32 x 32 x 16: PROBE_CHAINS / 2 instructions of four times the work
  const double per = shape == 16 ? PROBE_CHAINS * 16.0 * 16.0 * 32.0 * 2.0 : (PROBE_CHAINS / 2) * 32.0 * 32.0 * 16.0 * 2.0;
  return (double)blocks * 4.0 * iters * per;
}

int gdr_probe_read(const void* src, size_t bytes, int blocks, float* out, size_t out_elems, void* stream) {
  if (!src || !out || blocks < 1 || bytes % 16 || ((uintptr_t)src & 15) || (size_t)blocks * 256 > out_elems)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const f32x4*)src,
                     bytes / 16, out);
  return (int)hipGetLastError();
}

int gdr_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || blocks < 1 || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const f32x4*)src,
                     (f32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
