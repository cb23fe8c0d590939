// gdr_rmsnorm.hip -- fused RMSNorm backward (include/gdr_rmsnorm.h) on gfx950,
// with the weight-gradient reduction selectable between an in-kernel
// fixed-order (deterministic) reduction, floating-point atomics, and a
// separate fixed-order reduction kernel.  The in-kernel reduction of the
// workgroups' dw partials is the fusion Dao-AILab/quack PR #101 ("Rmsnorm
// backward fusing sum", description) makes; whether it must be
// deterministic is the question of that page's review thread.
//
// Per row (length N) with r = rstd or (mean x^2 + eps)^(-1/2), xhat = r x:
//   dx = r (w dy - xhat mean(w dy xhat)),   dw += dy xhat (summed over rows)
//
// Work split.  G workgroups of 256 threads each take a fixed contiguous
// range of rows (so every partial is the same whatever the scheduling).  A
// row is handled by TPR threads (64 = one wave, four rows at a time, or 256
// = the whole workgroup) holding EPT elements each in 16-byte pieces; the
// two row sums (x^2 when r is not given, w dy xhat) are butterfly sums
// inside a wave plus, for TPR = 256, a fixed-order sum of the four waves'
// values through LDS.  Each thread accumulates dw for its own columns in
// registers; the workgroup's partial is then reduced by the selected mode.
//
// Fixed-order mode, inside the kernel: each workgroup stores its partial,
// makes it visible at agent scope (a release fence, which writes the
// compute die's L2 back), then arrives on its group's counter (groups of
// 32 workgroups); the last to arrive -- whichever it is -- sums the group's
// partials in workgroup order, stores the group sum and arrives on the
// final counter; the last group to arrive sums the group sums in group
// order and adds them to dw.  The counters are returned to zero by the
// workgroups that consumed them.  No workgroup ever waits for another, so
// there is no dependence on which workgroups are resident.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>

#include "gdr_host.h"
#include "gdr_rmsnorm.h"

namespace {

constexpr int RN_GROUP = 32;          // workgroups per first-level group
constexpr int RN_MAX_WG = 1024;       // most workgroups (row partitions) per call
constexpr int RN_MIN_ROWS = 16;       // fewest rows per workgroup
constexpr int RN_COUNTERS = 512;      // bytes of counters at the start of the workspace (1 + 32 used)
static_assert((1 + RN_MAX_WG / RN_GROUP) * 4 <= RN_COUNTERS, "counters fit their region");
constexpr int RN_MAX_N = 8192;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a row (16 bytes of bf16, 32 of fp32) as fp32
template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
  static __device__ __forceinline__ void load(const __bf16* p, float* o) {
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    const b8 v = *reinterpret_cast<const b8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
  }
  static __device__ __forceinline__ void store(__bf16* p, const float* o) {
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    b8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)o[i];
    *reinterpret_cast<b8*>(p) = v;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = a[i];
      o[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* o) {
    *reinterpret_cast<f32x4*>(p) = (f32x4){o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(p + 4) = (f32x4){o[4], o[5], o[6], o[7]};
  }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

struct RnArgs {
  long M;
  int N;
  int G;              // workgroups = row partitions
  int mode;
  float eps;
  const void* x;
  const float* w;
  const void* dy;
  const float* rstd;  // nullable
  void* dx;
  float* dw;
  unsigned* cnt;      // [0]: final counter, [1 + grp]: group counters
  float* part;        // [G][N]: workgroup partials
  float* gpart;       // [ceil(G / RN_GROUP)][N]: group sums
};

// sum_{k < n} p[k * N .. + 3] in order k = 0, 1, ..., loads issued 8 rows
// at a time so that their latencies overlap
__device__ __forceinline__ f32x4 sum_rows_in_order(const float* p, int N, int n) {
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = k0 + u < n ? *reinterpret_cast<const f32x4*>(p + (long)(k0 + u) * N) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < n) acc += v[u];
  }
  return acc;
}

template <typename T, int TPR, int EPT>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const RnArgs a) {
  constexpr int RPI = 256 / TPR;   // rows in flight per workgroup
  constexpr int NV = EPT / 8;      // 8-element pieces per thread
  __shared__ __align__(16) float s_part[RN_MAX_N];   // the workgroup's dw partial
  __shared__ float s_red[2][4];
  __shared__ int s_last;
  const int tid = threadIdx.x, wv = tid >> 6;
  const int slot = tid / TPR, t = tid % TPR;
  const int N = a.N;
  const int g = blockIdx.x;
  const long rb = (long)g * a.M / a.G, re = (long)(g + 1) * a.M / a.G;
  const T* xp = (const T*)a.x;
  const T* dyp = (const T*)a.dy;
  T* dxp = (T*)a.dx;

  float wv8[EPT], dwp[EPT];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int c = (t + TPR * v) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wv8[8 * v + i] = c < N ? a.w[c + i] : 0.f;
      dwp[8 * v + i] = 0.f;
    }
  }
  const float invN = 1.0f / (float)N;
  int red = 0;   // reductions so far (selects the LDS buffer of a cross-wave sum)
  auto row_sum = [&](float s) {
    s = wave_sum(s);
    if constexpr (TPR == 256) {
      float* buf = s_red[red & 1];
      if ((tid & 63) == 0) buf[wv] = s;
      __syncthreads();
      s = ((buf[0] + buf[1]) + buf[2]) + buf[3];
      ++red;
    }
    return s;
  };

  // TPR = 256: every thread runs every row (uniform trip count, barriers
  // inside); TPR = 64: each wave runs its own rows, no barriers inside
  for (long row = rb + slot; row < re; row += RPI) {
    float xv[EPT], dyv[EPT];
    const long base = row * (long)N;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = (t + TPR * v) * 8;
      if (c < N) {
        Vec8<T>::load(xp + base + c, xv + 8 * v);
        Vec8<T>::load(dyp + base + c, dyv + 8 * v);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[8 * v + i] = dyv[8 * v + i] = 0.f;
      }
    }
    float r;
    if (a.rstd) {
      r = a.rstd[row];
    } else {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) ss += xv[i] * xv[i];
      r = 1.0f / sqrtf(row_sum(ss) * invN + a.eps);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) s += wv8[i] * dyv[i] * (xv[i] * r);
    const float cm = row_sum(s) * invN;
    float dxv[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const float xh = xv[i] * r;
      dxv[i] = r * (wv8[i] * dyv[i] - xh * cm);
      dwp[i] += dyv[i] * xh;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = (t + TPR * v) * 8;
      if (c < N) Vec8<T>::store(dxp + base + c, dxv + 8 * v);
    }
  }

  // the workgroup's partial in LDS: TPR = 256 owns every column once; with
  // TPR = 64 the four waves hold the same columns and add in wave order
  if constexpr (TPR == 256) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = (t + TPR * v) * 8;
      if (c < N)
#pragma unroll
        for (int i = 0; i < 8; ++i) s_part[c + i] = dwp[8 * v + i];
    }
    __syncthreads();
  } else {
    for (int k = 0; k < 4; ++k) {
      if (wv == k) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int c = (t + TPR * v) * 8;
          if (c < N)
#pragma unroll
            for (int i = 0; i < 8; ++i) s_part[c + i] = (k == 0 ? 0.f : s_part[c + i]) + dwp[8 * v + i];
        }
      }
      __syncthreads();
    }
  }

  if (a.mode == GDR_REDUCE_ATOMIC) {
    for (int c = tid; c < N; c += 256) unsafeAtomicAdd(a.dw + c, s_part[c]);
    return;
  }
  float* mine = a.part + (long)g * N;
  for (int c = 4 * tid; c < N; c += 1024)
    *reinterpret_cast<f32x4*>(mine + c) = *reinterpret_cast<const f32x4*>(s_part + c);
  if (a.mode == GDR_REDUCE_SEPARATE) return;

  // fixed-order mode.  The barrier completes every thread's stores of the
  // partial; the arrival is an agent-scope release (it writes the compute
  // die's L2 back, so the partial is visible to every die), and only the
  // last arriver takes the agent-scope acquire before reading the others'.
  const int grp = g / RN_GROUP;
  const int g0 = grp * RN_GROUP;
  const int members = min(RN_GROUP, a.G - g0);
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.cnt + 1 + grp, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(members - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int NG = (a.G + RN_GROUP - 1) / RN_GROUP;
  for (int c = 4 * tid; c < N; c += 1024)
    *reinterpret_cast<f32x4*>(a.gpart + (long)grp * N + c) = sum_rows_in_order(a.part + (long)g0 * N + c, N, members);
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_store(a.cnt + 1 + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned prev = __hip_atomic_fetch_add(a.cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(NG - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int c = 4 * tid; c < N; c += 1024) {
    f32x4* d = reinterpret_cast<f32x4*>(a.dw + c);
    *d = *d + sum_rows_in_order(a.gpart + c, N, NG);
  }
  if (tid == 0) __hip_atomic_store(a.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// separate mode, second kernel: dw[c] += sum over workgroups (in order);
// one thread per 4 columns
__global__ __launch_bounds__(256) void k_rmsnorm_reduce(const float* part, int G, int N, float* dw) {
  const int c = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (c >= N) return;
  f32x4* d = reinterpret_cast<f32x4*>(dw + c);
  *d = *d + sum_rows_in_order(part + c, N, G);
}

int workgroups(long M) {
  const long g = (M + RN_MIN_ROWS - 1) / RN_MIN_ROWS;
  return (int)(g < 1 ? 1 : (g > RN_MAX_WG ? RN_MAX_WG : g));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t part = 0, gpart = 0, total = 0;
};

Layout layout(long M, int N, int mode) {
  Layout l;
  if (mode == GDR_REDUCE_ATOMIC) return l;
  const int G = workgroups(M), NG = (G + RN_GROUP - 1) / RN_GROUP;
  l.part = RN_COUNTERS;
  l.gpart = align256(l.part + (size_t)G * N * 4);
  l.total = mode == GDR_REDUCE_FIXED ? align256(l.gpart + (size_t)NG * N * 4) : align256(l.gpart);
  return l;
}

bool bad_align(const void* p) { return ((uintptr_t)p & 15) != 0; }

template <typename T, int TPR, int EPT>
hipError_t launch(const RnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_rmsnorm_bwd<T, TPR, EPT>), dim3(a.G), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RnArgs& a, hipStream_t s) {
  if (a.N <= 512) return launch<T, 64, 8>(a, s);
  if (a.N <= 1024) return launch<T, 64, 16>(a, s);
  if (a.N <= 2048) return launch<T, 64, 32>(a, s);
  if (a.N <= 4096) return launch<T, 256, 16>(a, s);
  return launch<T, 256, 32>(a, s);
}

}  // namespace

extern "C" {

size_t gdr_rmsnorm_bwd_workspace_bytes(int M, int N, int mode) {
  if (M < 0 || N < 8 || N > RN_MAX_N || N % 8 || mode < 0 || mode > 2) return 0;
  return layout(M, N, mode).total;
}

gdr_status gdr_rmsnorm_bwd(int M, int N, int io_dtype, const void* x, const float* w, const void* dy,
                           const float* rstd, float eps, void* dx, float* dw, int mode, void* workspace,
                           size_t workspace_bytes, void* stream) {
  char msg[256];
  gdr::set_error("");
  if (M < 0 || N < 8 || N > RN_MAX_N || N % 8) {
    snprintf(msg, sizeof(msg), "need M >= 0 and N a multiple of 8 in [8, %d] (got M %d, N %d)", RN_MAX_N, M, N);
    gdr::set_error(msg);
    return GDR_ERR_UNSUPPORTED;
  }
  if (io_dtype != GDR_BF16 && io_dtype != GDR_F32) {
    gdr::set_error("io_dtype must be GDR_BF16 or GDR_F32");
    return GDR_ERR_UNSUPPORTED;
  }
  if (mode < GDR_REDUCE_FIXED || mode > GDR_REDUCE_SEPARATE) {
    gdr::set_error("mode must be GDR_REDUCE_FIXED, GDR_REDUCE_ATOMIC or GDR_REDUCE_SEPARATE");
    return GDR_ERR_INVALID_ARG;
  }
  if (!rstd && !(eps >= 0.f && std::isfinite(eps))) {
    gdr::set_error("eps must be finite and >= 0 when rstd is not given");
    return GDR_ERR_INVALID_ARG;
  }
  if (M == 0) return GDR_OK;   // no rows: dw unchanged, nothing to launch
  if (!x || !w || !dy || !dx || !dw) {
    gdr::set_error("x, w, dy, dx and dw are required");
    return GDR_ERR_INVALID_ARG;
  }
  const void* ptrs[] = {x, w, dy, dx, dw, workspace};
  for (const void* p : ptrs)
    if (p && bad_align(p)) {
      gdr::set_error("x, w, dy, dx, dw and the workspace must be 16-byte aligned");
      return GDR_ERR_INVALID_ARG;
    }
  if (rstd && ((uintptr_t)rstd & 3)) {
    gdr::set_error("rstd must be 4-byte aligned");
    return GDR_ERR_INVALID_ARG;
  }
  const Layout l = layout(M, N, mode);
  char* ws = (char*)workspace;
  if (mode != GDR_REDUCE_ATOMIC) {
    if (!ws || workspace_bytes < l.total || ((uintptr_t)ws & 255)) {
      snprintf(msg, sizeof(msg), "a 256-byte aligned workspace of %zu bytes is needed (got %zu)", l.total,
               ws ? workspace_bytes : (size_t)0);
      gdr::set_error(msg);
      return GDR_ERR_WORKSPACE;
    }
  }
  RnArgs a{};
  a.M = M; a.N = N; a.G = workgroups(M); a.mode = mode; a.eps = eps;
  a.x = x; a.w = w; a.dy = dy; a.rstd = rstd; a.dx = dx; a.dw = dw;
  a.cnt = ws ? (unsigned*)ws : nullptr;
  a.part = ws ? (float*)(ws + l.part) : nullptr;
  a.gpart = ws ? (float*)(ws + l.gpart) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = io_dtype == GDR_BF16 ? launch_t<__bf16>(a, s) : launch_t<float>(a, s);
  if (e == hipSuccess && mode == GDR_REDUCE_SEPARATE) {
    hipLaunchKernelGGL(k_rmsnorm_reduce, dim3((N / 4 + 255) / 256), dim3(256), 0, s, (const float*)a.part, a.G, N, dw);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "launch failed: %s", hipGetErrorString(e));
    gdr::set_error(msg);
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

}  // extern "C"
