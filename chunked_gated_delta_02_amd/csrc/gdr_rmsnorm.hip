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
#ifdef GDR_DEBUG_DELAY
#include "gdr_kernels.h"   // the race-test build's delay hook (gdr_device.h)
#endif

namespace {

// Barriers, and the points around the cross-workgroup hand-offs of the
// fixed-order reduction, where the race-test build (GDR_DEBUG_DELAY) can put
// chosen waves to sleep; in the production build RN_DELAY is empty.
#ifdef GDR_DEBUG_DELAY
#define RN_DELAY() ::gdr::debug_delay()
#else
#define RN_DELAY() \
  do {             \
  } while (0)
#endif
#define RN_SYNC()    \
  do {               \
    __syncthreads(); \
    RN_DELAY();      \
  } while (0)

constexpr int RN_GROUP = 32;          // workgroups per first-level group
constexpr int RN_MAX_WG = 512;        // most workgroups (row partitions) per call
constexpr int RN_MIN_ROWS = 16;       // fewest rows per workgroup
constexpr int RN_COUNTERS = 512;      // bytes of counters at the start of the workspace (1 + 32 used)
static_assert((1 + RN_MAX_WG / RN_GROUP) * 4 <= RN_COUNTERS, "counters fit their region");
constexpr int RN_MAX_N = 8192;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a row (16 bytes of bf16, 32 of fp32), held as
// loaded (so a prefetched row costs its raw size in registers) and widened
// to fp32 where used.  Every element of x and dy is read once and every
// element of dx written once, so the bf16 rows move with streaming
// (non-temporal) loads and stores: measured 5-25 % faster than cached ones
// across the sweep, and at M = 65536, N = 8192 at the rate of a plain copy.
template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
  typedef __bf16 b8 __attribute__((ext_vector_type(8)));
  b8 d;
  __device__ __forceinline__ void load(const __bf16* p) { d = __builtin_nontemporal_load(reinterpret_cast<const b8*>(p)); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = (__bf16)0.f;
  }
  __device__ __forceinline__ float operator[](int i) const { return (float)d[i]; }
  static __device__ __forceinline__ void store(__bf16* p, const float* o) {
    b8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)o[i];
    __builtin_nontemporal_store(v, reinterpret_cast<b8*>(p));
  }
};
template <> struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = (f32x4){0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
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

// For the NC column pieces c = c0 + j * cstride (j < NC, 4 columns each,
// those >= N skipped): out[j] = sum_{k < n} p[k * N + c .. + 3], added in
// order k = 0, 1, ....  Loads are issued RB rows at a time for all NC pieces
// together, so NC * RB loads per thread are in flight (one workgroup reading
// a few MB on its own is bound by what it keeps in flight).
template <int NC, int RB = 8>
__device__ __forceinline__ void sum_rows_in_order(const float* p, int N, int n, int c0, int cstride, f32x4* out) {
#pragma unroll
  for (int j = 0; j < NC; ++j) out[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += RB) {
    f32x4 v[NC][RB];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int c = c0 + j * cstride;
        v[j][u] = (k0 + u < n && c < N) ? *reinterpret_cast<const f32x4*>(p + (long)(k0 + u) * N + c)
                                        : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int j = 0; j < NC; ++j)
        if (k0 + u < n) out[j] += v[j][u];
  }
}

// dst[c] (+)= ordered sum over n rows of p, for every column piece of the
// workgroup (NT threads, 4 columns per thread and piece)
template <int NT, bool ADD>
__device__ __forceinline__ void reduce_rows(const float* p, int N, int n, float* dst) {
  constexpr int NC = 2;   // 16 loads in flight per thread; more would raise the kernel's register count
  for (int cb = 4 * (int)threadIdx.x; cb < N; cb += NC * 4 * NT) {
    f32x4 acc[NC];
    sum_rows_in_order<NC>(p, N, n, cb, 4 * NT, acc);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = cb + j * 4 * NT;
      if (c < N) {
        f32x4* d = reinterpret_cast<f32x4*>(dst + c);
        *d = ADD ? *d + acc[j] : acc[j];
      }
    }
  }
}

template <typename T, int NT, int TPR, int EPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && EPT <= 16 ? 4 : 2, 8))) void k_rmsnorm_bwd(const RnArgs a) {
  static_assert(TPR == 64 || TPR == NT, "a row is one wave or the whole workgroup");
  constexpr int NW = NT / 64;      // waves
  constexpr int RPI = NT / TPR;    // rows in flight per workgroup
  constexpr int NV = EPT / 8;      // 8-element pieces per thread
  extern __shared__ __align__(16) float s_part[];   // [N]: the workgroup's dw partial
  __shared__ float s_red[2][NW];
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
    if constexpr (TPR == NT && NW > 1) {
      float* buf = s_red[red & 1];
      if ((tid & 63) == 0) buf[wv] = s;
      RN_SYNC();
      s = buf[0];
#pragma unroll
      for (int k = 1; k < NW; ++k) s += buf[k];
      ++red;
    }
    return s;
  };

  // One row ahead: the next row's x and dy (and rstd) are loaded while the
  // current one is computed.  TPR = NT: every thread runs every row (uniform
  // trip count, barriers inside); TPR = 64: each wave runs its own rows.
  Vec8<T> xr[NV], dr[NV];
  float rr = 0.f;
  auto issue = [&](long row) {
    const long base = row * (long)N;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = (t + TPR * v) * 8;
      if (c < N) {
        xr[v].load(xp + base + c);
        dr[v].load(dyp + base + c);
      } else {
        xr[v].zero();
        dr[v].zero();
      }
    }
    if (a.rstd) rr = a.rstd[row];
  };
  long row = rb + slot;
  if (row < re) issue(row);
  for (; row < re; row += RPI) {
    float xv[EPT], dyv[EPT];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xv[8 * v + i] = xr[v][i];
        dyv[8 * v + i] = dr[v][i];
      }
    float r = rr;
    if (row + RPI < re) issue(row + RPI);
    if (!a.rstd) {
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
    const long base = row * (long)N;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = (t + TPR * v) * 8;
      if (c < N) Vec8<T>::store(dxp + base + c, dxv + 8 * v);
    }
  }

  // the workgroup's partial in LDS: TPR = NT owns every column once; with
  // TPR = 64 the waves hold the same columns and add in wave order
  if constexpr (TPR == NT) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = (t + TPR * v) * 8;
      if (c < N)
#pragma unroll
        for (int i = 0; i < 8; ++i) s_part[c + i] = dwp[8 * v + i];
    }
    RN_SYNC();
  } else {
    for (int k = 0; k < NW; ++k) {
      if (wv == k) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int c = (t + TPR * v) * 8;
          if (c < N)
#pragma unroll
            for (int i = 0; i < 8; ++i) s_part[c + i] = (k == 0 ? 0.f : s_part[c + i]) + dwp[8 * v + i];
        }
      }
      RN_SYNC();
    }
  }

  if (a.mode == GDR_REDUCE_ATOMIC) {
    for (int c = tid; c < N; c += NT) unsafeAtomicAdd(a.dw + c, s_part[c]);
    return;
  }
  float* mine = a.part + (long)g * N;
  RN_DELAY();
  for (int c = 4 * tid; c < N; c += 4 * NT)
    *reinterpret_cast<f32x4*>(mine + c) = *reinterpret_cast<const f32x4*>(s_part + c);
  if (a.mode == GDR_REDUCE_SEPARATE) return;

  // fixed-order mode.  The barrier completes every thread's stores of the
  // partial; the arrival is an agent-scope release (it writes the compute
  // die's L2 back, so the partial is visible to every die), and only the
  // last arriver takes the agent-scope acquire before reading the others'.
  const int grp = g / RN_GROUP;
  const int g0 = grp * RN_GROUP;
  const int members = min(RN_GROUP, a.G - g0);
  RN_SYNC();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.cnt + 1 + grp, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(members - 1);
  }
  RN_SYNC();
  if (!s_last) return;
  RN_DELAY();
  __threadfence();
  const int NG = (a.G + RN_GROUP - 1) / RN_GROUP;
  reduce_rows<NT, false>(a.part + (long)g0 * N, N, members, a.gpart + (long)grp * N);
  RN_SYNC();
  if (tid == 0) {
    __hip_atomic_store(a.cnt + 1 + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned prev = __hip_atomic_fetch_add(a.cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(NG - 1);
  }
  RN_SYNC();
  if (!s_last) return;
  RN_DELAY();
  __threadfence();
  reduce_rows<NT, true>(a.gpart, N, NG, a.dw);
  if (tid == 0) __hip_atomic_store(a.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// separate mode, second kernel: dw[c] += sum over workgroups (in order);
// 4 columns per thread and piece, RN_RED_COLS columns per workgroup
constexpr int RN_RED_COLS = 256;
__global__ __launch_bounds__(64) void k_rmsnorm_reduce(const float* part, int G, int N, float* dw) {
  const int c = blockIdx.x * RN_RED_COLS + 4 * (int)threadIdx.x;
  f32x4 acc;
  sum_rows_in_order<1, 16>(part, N, G, c, 0, &acc);
  if (c < N) {
    f32x4* d = reinterpret_cast<f32x4*>(dw + c);
    *d = *d + acc;
  }
}

// Workgroups (row partitions): at least RN_MIN_ROWS rows each, and at most
// one per compute unit (256 on MI355X) -- or two where a row of N <= 2048 is
// spread over the whole workgroup, whose barrier per row a second workgroup
// on the CU hides.  Fewer partials shorten the fixed-order reduction at the
// end, and one workgroup per CU already keeps enough rows in flight (with
// the one-row prefetch) for the rest; measured over the sweep against caps
// of 384, 512 and 1024.
int workgroups(long M, int N) {
  const long cap = (N > 1024 && N <= 2048) ? 512 : 256;
  const long g = (M + RN_MIN_ROWS - 1) / RN_MIN_ROWS;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t part = 0, gpart = 0, total = 0;
};

Layout layout(long M, int N, int mode) {
  Layout l;
  if (mode == GDR_REDUCE_ATOMIC) return l;
  const int G = workgroups(M, N), NG = (G + RN_GROUP - 1) / RN_GROUP;
  l.part = RN_COUNTERS;
  l.gpart = align256(l.part + (size_t)G * N * 4);
  l.total = mode == GDR_REDUCE_FIXED ? align256(l.gpart + (size_t)NG * N * 4) : align256(l.gpart);
  return l;
}

bool bad_align(const void* p) { return ((uintptr_t)p & 15) != 0; }

template <typename T, int NT, int TPR, int EPT>
hipError_t launch(const RnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_rmsnorm_bwd<T, NT, TPR, EPT>), dim3(a.G), dim3(NT), (size_t)a.N * sizeof(float), s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RnArgs& a, hipStream_t s) {
  if (a.N <= 512) return launch<T, 256, 64, 8>(a, s);
  if (a.N <= 1024) return launch<T, 256, 64, 16>(a, s);
  if (a.N <= 2048) return launch<T, 256, 256, 8>(a, s);
  if (a.N <= 4096) return launch<T, 256, 256, 16>(a, s);
  return launch<T, 256, 256, 32>(a, s);
}

}  // namespace

#ifdef GDR_DEBUG_DELAY
namespace gdr {
// the race-test build: this file's copy of the barrier-delay settings
hipError_t debug_set_delay_rmsnorm(const DelayCfg& c) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_delay), &c, sizeof(c));
}
}  // namespace gdr
#endif

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
  a.M = M; a.N = N; a.G = workgroups(M, N); a.mode = mode; a.eps = eps;
  a.x = x; a.w = w; a.dy = dy; a.rstd = rstd; a.dx = dx; a.dw = dw;
  a.cnt = ws ? (unsigned*)ws : nullptr;
  a.part = ws ? (float*)(ws + l.part) : nullptr;
  a.gpart = ws ? (float*)(ws + l.gpart) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = io_dtype == GDR_BF16 ? launch_t<__bf16>(a, s) : launch_t<float>(a, s);
  if (e == hipSuccess && mode == GDR_REDUCE_SEPARATE) {
    hipLaunchKernelGGL(k_rmsnorm_reduce, dim3((N + RN_RED_COLS - 1) / RN_RED_COLS), dim3(64), 0, s, (const float*)a.part, a.G, N, dw);
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
