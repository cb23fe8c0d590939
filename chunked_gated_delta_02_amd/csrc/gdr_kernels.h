// gdr_kernels.h -- kernel argument blocks, LDS staging helpers and launcher
// declarations shared by the forward and backward kernel files.
#pragma once

#include "gdr_device.h"
#include "libgdr.h"

#define GDR_MAX_SEQS 8192

// per chunk-head gate block in the workspace: gamma[64] (hi), e^gamma[64],
// e^{gamma_L - gamma}[64]; the lo part of gamma (gamma = hi + lo, an exact
// two-float sum) lives in an array of its own, 64 per chunk-head, at the end
// of the workspace
#define GSTRIDE 192


namespace gdr {

// LDS row padding in elements: 16 bytes for 16-bit tiles (keeps 16-byte
// aligned rows for ds_read_b128 and shifts consecutive rows by 4 banks),
// 16 bytes for fp32 tiles as well.
template <typename T> constexpr int pad_of() { return sizeof(T) == 2 ? 8 : 4; }
// value-dim block processed at once by the chunk-parallel kernels
template <typename T> constexpr int dvb_of() { return sizeof(T) == 2 ? 64 : 32; }
constexpr int cmax(int x, int y) { return x > y ? x : y; }

// Workspace tensors are head-major, [H][slot][...], so the chunks of one
// (sequence, head) are contiguous.  Operands the scans and the gradient
// kernel feed to MFMA are stored in fragment order (afrag<R, K>: a wave's
// fragment is one contiguous 1 KB block) and per-tile results in
// accumulator order (acc<R, C>), so every access of the serial scans is a
// fully coalesced wave-wide load or store.
// Operands are exact copies of the inputs wherever possible; where an
// MFMA operand is a computed value whose bf16 rounding would dominate the
// error (P, scale Q~^T), it is stored split (hi and lo).  Values the scans
// add to their accumulators (U, scale P^T dO, scale Q~^T dO) are fp32.
struct WyArgs {
  Geo geo;
  int DV;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const void* dO;    // backward only
  const float* beta;
  const float* g;
  float* gam;   // [GSTRIDE]: gamma (hi), e^gamma, e^{gamma_L - gamma}
  float* gaml;  // [64]: gamma (lo)
  void* Wf;     // afrag<64, DK>: W (rows r, k = dk); backward: nullable
  float* Ua;    // acc<64, DV> fp32: U; backward: nullable
  void* KtTf;   // afrag<DK, 64>: K^T (exact; nullable)
  void* Qf;     // afrag<64, DK>: Q (exact)                          (forward)
  void* Pf;     // afrag<64, 64>: P = Q K^T * Gam (rows r), hi part  (forward)
  void* Pfl;    // the lo part (bf16 only)                           (forward)
  float* Tm;    // [64][64] row-major fp32: T                        (backward)
  void* WTf;    // afrag<DK, 64>: W^T                                (backward)
  void* Kf;     // afrag<64, DK>: K (exact)                          (backward)
  float* dDl;   // acc<64, DV> fp32: scale P^T dO                    (backward)
  float* Z;     // acc<DK, DV> fp32: scale (e^gamma Q)^T dO          (backward)
};

// The serial scans run one workgroup per (unit, column tile); a unit is a
// (sequence, CP segment, head).  In the CP summary mode (MODE 0) the columns
// are those of the augmented state [transition | state from zero], DK + DV
// wide; otherwise the DV columns of the state.
struct ScanFwdArgs {
  Geo geo;
  int DV;
  int ntiles;        // column tiles per unit (set by the launcher)
  int layout;        // 0: KV, 1: VK for h0 / hT
  float scale;
  const float* h0;   // nullable
  float* hT;         // nullable
  const float* hstart;  // CP: [cp][N][H][DK][DV] fp32 start state of each segment (s >= 1)
  float* summ;          // CP summary out: [cp][N][H][DK][DK + DV] fp32 (s < cp - 1)
  const float* gam;
  const void* Wf;
  const void* KtTf;
  const float* Ua;
  const void* Qf;    // output operands (MODE 2)
  const void* Pf;
  const void* Pfl;
  void* o;
  void* hs;          // acc<DK, DV> per chunk-head: state at chunk start (MODE 1, 2)
};

struct ScanBwdArgs {
  Geo geo;
  int DV;
  int ntiles;
  int layout;
  const float* dhT;  // nullable
  float* dh0;        // nullable
  const float* dhend;   // CP: [cp][N][H][DK][DV] fp32 gradient at each segment's end (s < cp - 1)
  float* summ;          // CP summary out: [cp][N][H][DK][DK + DV] fp32 (s >= 1)
  const float* gam;
  const void* Kf;
  const void* WTf;
  const float* dDl;
  const float* Z;
  void* dhs;         // acc<DK, DV> (io dtype): gradient of the state at chunk end
  void* dD;          // acc<64, DV> (io dtype): gradient of Delta
};

// Hand-off of the CP segment states, per (sequence, head, 64-column tile):
// forward, h_start[s + 1] = M_s h_start[s] + b_s from h_start[0] = h0;
// backward, dh_end[s - 1] = X_s dh_end[s] + d_s from dh_end[cp - 1] = dh_T,
// with [M_s | b_s] / [X_s | d_s] the segment summaries.
struct CpChainArgs {
  Geo geo;             // N, H, cp
  int DK, DV;
  int layout;          // of init
  int bwd;
  const float* init;   // h0 (forward) / dh_T (backward), user layout; nullable (zeros)
  const float* summ;   // [cp][N][H][DK][DK + DV]
  float* out;          // [cp][N][H][DK][DV]: h_start (forward) / dh_end (backward)
};

struct GradArgs {
  Geo geo;
  int DV;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* beta;
  const float* gam;
  const float* gaml;    // [64] per chunk-head: gamma (lo)
  const void* WTf;      // afrag<DK, 64>: W^T
  const float* Tm;      // [64][64] row-major fp32: T
  const void* hs;
  const void* dhs;
  const void* dD;
  void* dq;
  void* dk;
  void* dv;
  float* dbeta;
  float* dg;
};

// ---------------------------------------------------------------------------
// LDS staging (workgroups of NTHR threads, 256 unless stated).  NR rows of NC elements from
// global (row stride gstride elements) into LDS (row stride ld); rows >=
// nvalid are zero.  16-byte accesses.  All of a thread's loads are issued
// before its first LDS store (compile-time trip count), so their latencies
// overlap instead of adding up.
template <typename T, int NC, int NR = 64, int NTHR = 256>
struct RowBuf {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int PER_ROW = NC / VEC;
  static constexpr int NP = NR * PER_ROW;
  static constexpr int IT = (NP + NTHR - 1) / NTHR;
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 v[IT];
  // issue the loads (registers only); rows >= nvalid read as zero through
  // the buffer range check
  __device__ __forceinline__ void load(const T* g, int64_t gstride, int nvalid) {
    static_assert(NP % NTHR == 0, "whole trips only");
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(g, nvalid * (int)gstride * (int)sizeof(T));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = threadIdx.x + NTHR * it;
      const int r = e / PER_ROW, c = (e - r * PER_ROW) * VEC;
      v[it] = buf_load16(rs, (r * (int)gstride + c) * (int)sizeof(T));
    }
  }
  // write them to LDS
  __device__ __forceinline__ void store(T* s, int ld) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = threadIdx.x + NTHR * it;
      const int r = e / PER_ROW, c = (e - r * PER_ROW) * VEC;
      if (e < NP) *reinterpret_cast<f4*>(s + r * ld + c) = v[it];
    }
  }
};

template <typename T, int NC, int NR = 64, int NTHR = 256>
__device__ __forceinline__ void load_rows(T* s, int ld, const T* g, int64_t gstride, int nvalid) {
  RowBuf<T, NC, NR, NTHR> b;
  b.load(g, gstride, nvalid);
  b.store(s, ld);
}

// Copy an R x K matrix from LDS into afrag<R, K> order, one MFMA fragment
// (64 lanes x 16 bytes for bf16) per wave step: element (i, k) is
// src[i * ld + k] (RowK) or src[k * ld + i] (ColK).  4 waves.
template <typename T, int R, int K, bool COLK>
__device__ __forceinline__ void copy_afrag(T* dst, const T* src, int ld) {
  constexpr int KW = Mma<T>::KW, KPL = Mma<T>::KPL;
  constexpr int NF = (R / 16) * (K / KW);
  typedef typename Mma<T>::frag frag;
#pragma unroll
  for (int f = wave_id(); f < NF; f += 4) {
    const int m = f / (K / KW), s = f - m * (K / KW);
    const frag v = COLK ? frag_colk_lds(src, ld, 16 * m, s * KW) : frag_rowk(src, ld, 16 * m, s * KW);
    *reinterpret_cast<frag*>(dst + ((int64_t)f * 64 + lane_id()) * KPL) = v;
  }
}

// Same for an fp32 LDS matrix (RowK, row stride ld, 16-byte aligned rows)
// written as a split pair: hi into dst, lo into dlo (fp32 operands: dst only).
template <typename T, int R, int K>
__device__ __forceinline__ void copy_afrag_split(T* dst, T* dlo, const float* src, int ld) {
  constexpr int KW = Mma<T>::KW, KPL = Mma<T>::KPL;
  constexpr int NF = (R / 16) * (K / KW);
  typedef typename Mma<T>::frag frag;
  auto one = [](int) { return 1.f; };
#pragma unroll
  for (int f = wave_id(); f < NF; f += 4) {
    const int m = f / (K / KW), s = f - m * (K / KW);
    frag hi, lo;
    frag_rowk_f32<T>(src, ld, 16 * m, s * KW, one, hi, lo);
    *reinterpret_cast<frag*>(dst + ((int64_t)f * 64 + lane_id()) * KPL) = hi;
    if constexpr (sizeof(T) == 2) *reinterpret_cast<frag*>(dlo + ((int64_t)f * 64 + lane_id()) * KPL) = lo;
  }
}

template <typename T>
__device__ __forceinline__ f32x4 load4f(const T* p) {
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    const t4 v = *reinterpret_cast<const t4*>(p);
    return (f32x4){to_f32(v[0]), to_f32(v[1]), to_f32(v[2]), to_f32(v[3])};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

// Transposed accumulator tiles.  With the operands of C = A B swapped,
// Mma<T>::mma(b, a, c) accumulates (A B)^T: the A and B fragments use the
// same map of lanes, so nothing moves.  Lane l then holds row tr_row() of
// A B and its four consecutive columns tr_col0() .. + 3 (relative to the
// tile): one 8- or 16-byte piece of a row, stored or scaled per row with no
// cross-lane exchange.
__device__ __forceinline__ int tr_row() { return lane_id() & 15; }
__device__ __forceinline__ int tr_col0() { return 4 * (lane_id() >> 4); }

// Four consecutive elements of type T at byte offset voff + soff of a buffer
// (one 8-byte store for 16-bit T, 16 bytes for fp32).  As for buf_store1,
// the row part of the offset must be in voff, which the range check sees.
template <typename T>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, f32x4 v, int voff, int soff) {
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const t4 w = {from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), r, voff, soff, 0);
  } else {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 0);
  }
}

// launchers (return the HIP error of the launch)
hipError_t launch_plan(const int* cu, int N, int T_total, int nchunks, int* seq_chunk, int* chunk_seq,
                       hipStream_t st);
hipError_t launch_check_cu(const int* cu, int N, int T_total, int* result, hipStream_t st);
hipError_t launch_wy(const WyArgs& a, bool f32, int DK, bool bwd, hipStream_t st);
// mode 0: CP segment summaries; forward 1: snapshots only, 2: snapshots and
// output; backward 1: the reverse scan proper
hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool f32, int hs_dtype, int DK, int dvt, int mode, hipStream_t st);
hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool f32, int DK, int dvt, int mode, hipStream_t st);
hipError_t launch_cp_chain(const CpChainArgs& a, hipStream_t st);
hipError_t launch_grad(const GradArgs& a, bool f32, int hs_dtype, int DK, hipStream_t st);
#ifdef GDR_DEBUG_DELAY
// barrier-delay settings of the kernels in each source file (race-test build)
hipError_t debug_set_delay_fwd(const DelayCfg& c);
hipError_t debug_set_delay_bwd(const DelayCfg& c);
hipError_t debug_set_delay_rmsnorm(const DelayCfg& c);
#endif

}  // namespace gdr
