// gdr_device.h -- device-side building blocks for the gfx950 (CDNA4) kernels
// of the chunked gated delta rule: MFMA wrappers, operand-fragment loads from
// LDS and global memory, accumulator-tile element maps, wavefront scans and
// the chunk geometry of fixed-length and packed variable-length batches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef __bf16 bf16;

#define GDR_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int lane_id() { return __lane_id(); }
// wave index within the workgroup, as a wave-uniform (scalar) value: the
// compiler then keeps it and what is derived from it in scalar registers and
// branches on it without execution masks
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// element conversions

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

// ---------------------------------------------------------------------------
// MFMA: 16x16 output tiles.  Lane l supplies A[row l&15][k-slice(l>>4)] and
// B[k-slice(l>>4)][col l&15]; the fp32 result holds C[4*(l>>4)+i][l&15].
// bf16 operands use v_mfma_f32_16x16x32_bf16 (8 k per lane), fp32 operands
// v_mfma_f32_16x16x4_f32 (1 k per lane).

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KW = 32;   // k per instruction
  static constexpr int KPL = 8;   // k per lane
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag neg(frag a) {
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    u16x8 u = __builtin_bit_cast(u16x8, a);
    u ^= (unsigned short)0x8000;
    return __builtin_bit_cast(frag, u);
  }
  static __device__ __forceinline__ frag zero() {
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(frag, (u16x8)(unsigned short)0);
  }
};
template <> struct Mma<float> {
  static constexpr int KW = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag neg(frag a) { return -a; }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
};

__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Operand fragments.
//
// "RowK" view: element (i, k) lives at p[i * ld + k] (k contiguous).
// "ColK" view: element (i, k) lives at p[k * ld + i] (i contiguous).
// A fragment for rows i0..i0+15 and k-block k0..k0+KW-1 gives lane l the
// elements (i0 + (l & 15), k0 + KPL*(l >> 4) + j), j < KPL.

// RowK from LDS or global: bf16 -> one 16-byte load.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_rowk(const T* p, int ld, int i0, int k0) {
  const int l = lane_id();
  const T* q = p + (int64_t)(i0 + (l & 15)) * ld + k0 + Mma<T>::KPL * (l >> 4);
  if constexpr (Mma<T>::KPL == 8) {
    return *reinterpret_cast<const bf16x8*>(q);
  } else {
    return *q;
  }
}

// Raw buffer resource over the bytes [p, p + bytes).  The hardware range
// check of raw buffers (stride 0) makes loads past the end return zero and
// drops stores past it, so a chunk's rows beyond its length need no branch:
// with p at the chunk's first row and bytes = length x row stride, exactly
// the rows past the length fall outside.  Offsets are 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// RowK fragment from a buffer (element offsets; ld = row stride in elements)
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_rowk_buf(__amdgpu_buffer_rsrc_t r, int ld, int i0, int k0) {
  const int l = lane_id();
  const int off = ((i0 + (l & 15)) * ld + k0 + Mma<T>::KPL * (l >> 4)) * (int)sizeof(T);
  if constexpr (Mma<T>::KPL == 8) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
}

// 16 bytes from a buffer at byte offset off
__device__ __forceinline__ f32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One element of type T to a buffer at byte offset voff + soff.  The row
// part of an offset must be in voff, the per-lane offset: it decides the
// range check (soff, a uniform offset inside the row, cannot move a store
// across a row boundary).
template <typename T>
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, float x, int voff, int soff) {
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f32<T>(x)), r, voff, soff, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, voff, soff, 0);
  }
}

// ColK from LDS.  bf16 uses the gfx950 transposing LDS read
// ds_read_b64_tr_b16: within each 16-lane group, lane j addresses the 4
// contiguous elements at (row j>>2, cols 4*(j&3)..+3) of a 4 x 16 block and
// lane i receives column i of that block (4 consecutive rows).  Two such
// reads give the 8 k values of a bf16 fragment.  Requires ld % 4 == 0 and
// i0 % 4 == 0 (8-byte aligned addresses).
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_colk_lds(const T* p, int ld, int i0, int k0) {
  const int l = lane_id();
  if constexpr (Mma<T>::KPL == 8) {
    const int j = l & 15;
    const int kb = k0 + 8 * (l >> 4) + (j >> 2);
    const int ib = i0 + 4 * (j & 3);
    const GDR_LDS i16x4* a0 = (const GDR_LDS i16x4*)((const GDR_LDS T*)p + kb * ld + ib);
    const GDR_LDS i16x4* a1 = (const GDR_LDS i16x4*)((const GDR_LDS T*)p + (kb + 4) * ld + ib);
    i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS i16x4*)a0);
    i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS i16x4*)a1);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 r = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
  } else {
    return p[(k0 + (l >> 4)) * ld + i0 + (l & 15)];
  }
}

// The lane's accumulator-layout elements (rows r0 + acc_row0() + i, column
// c0 + acc_col()) of a row-major LDS tile.  16-bit tiles take one
// transposing read per 16 x 16 tile: 16-lane group g reads the 4 x 16 block
// at rows r0 + 4g, lane j addressing (row j>>2, cols 4(j&3)..+3), and lane j
// receives column j of the block -- its 4 accumulator rows.  The values stay
// in the tile's type until read (operator[] converts to fp32).  Requires
// ld % 4 == 0 and c0 % 4 == 0.
template <typename T> struct AccVals {
  i16x4 v;
  // the whole vector is reinterpreted at once: a bit cast of a single
  // element of a short vector to a 16-bit float type is miscompiled here
  // (every element then reads element 0)
  __device__ __forceinline__ float operator[](int i) const {
    typedef T t4 __attribute__((ext_vector_type(4)));
    return to_f32(__builtin_bit_cast(t4, v)[i]);
  }
};
template <> struct AccVals<float> {
  f32x4 v;
  __device__ __forceinline__ float operator[](int i) const { return v[i]; }
};
template <typename T>
__device__ __forceinline__ AccVals<T> lds_acc(const T* p, int ld, int r0, int c0) {
  const int l = lane_id();
  AccVals<T> r;
  if constexpr (sizeof(T) == 2) {
    const int j = l & 15;
    const GDR_LDS i16x4* a0 =
        (const GDR_LDS i16x4*)((const GDR_LDS T*)p + (r0 + 4 * (l >> 4) + (j >> 2)) * ld + c0 + 4 * (j & 3));
    r.v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDR_LDS i16x4*)a0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = p[(r0 + 4 * (l >> 4) + i) * ld + c0 + (l & 15)];
  }
  return r;
}

// ---------------------------------------------------------------------------
// Fragment order ("afrag"): an R x K operand matrix (rows i, contraction
// index k) stored so that the fragment of row tile m and k-step s -- what
// one wave feeds to one MFMA -- is 64 lanes x KPL contiguous elements.  A
// wave loads a fragment with one fully coalesced access (1 KB for bf16).
template <typename T, int K>
__device__ __forceinline__ int64_t afrag_off(int i, int k) {
  constexpr int KW = Mma<T>::KW, KPL = Mma<T>::KPL;
  const int lane = (i & 15) + 16 * ((k % KW) / KPL);
  return ((int64_t)((i >> 4) * (K / KW) + k / KW) * 64 + lane) * KPL + (k % KPL);
}
template <typename T, int K>
__device__ __forceinline__ typename Mma<T>::frag frag_af(const T* p, int m, int s) {
  const T* q = p + ((int64_t)(m * (K / Mma<T>::KW) + s) * 64 + lane_id()) * Mma<T>::KPL;
  return *reinterpret_cast<const typename Mma<T>::frag*>(q);
}

// Accumulator order ("acc"): an R x C matrix stored so that 16 x 16 tile
// (m, n) is 64 lanes x 4 contiguous elements in the MFMA result layout
// (lane l holds rows 16m + 4(l>>4) + i, column 16n + (l&15)).
__device__ __forceinline__ int64_t acc_off(int m, int n, int C) {
  return ((int64_t)(m * (C / 16) + n) * 64 + lane_id()) * 4;
}
__device__ __forceinline__ int64_t acc_off_l(int m, int n, int C, int l) {
  return ((int64_t)(m * (C / 16) + n) * 64 + l) * 4;
}

// ---------------------------------------------------------------------------
// Accumulator tile element map: lane l holds C[r0 + i][c], i < 4, with
// r0 = 4*(l>>4), c = l & 15 (relative to the tile origin).
__device__ __forceinline__ int acc_row0() { return 4 * (lane_id() >> 4); }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

// Byte offsets of the lane's 4 accumulator rows (rows r0 + acc_row0() + i,
// column acc_col()) in a buffer of rows with stride ld elements of size sz
struct AccRows {
  int off[4];
};
__device__ __forceinline__ AccRows acc_rows(int ld, int r0, int sz) {
  AccRows a;
  const int o = ((r0 + acc_row0()) * ld + acc_col()) * sz;
#pragma unroll
  for (int i = 0; i < 4; ++i) a.off[i] = o + i * ld * sz;
  return a;
}

// An accumulator tile to the buffer rows of ar, starting at column c0 (the
// column offset goes in the uniform offset)
template <typename T>
__device__ __forceinline__ void buf_store_acc(__amdgpu_buffer_rsrc_t r, const AccRows& ar, int c0, f32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) buf_store1<T>(r, v[i], ar.off[i], c0 * (int)sizeof(T));
}


// Store an accumulator tile transposed: dst[(c0 + c) * ld + (r0 + r0l + i)],
// i.e. the 4 consecutive rows of the lane become 4 contiguous elements.
template <typename T>
__device__ __forceinline__ void store_acc_t(T* dst, int ld, int r0, int c0, f32x4 v) {
  T* q = dst + (int64_t)(c0 + acc_col()) * ld + r0 + acc_row0();
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 w = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
    *reinterpret_cast<t4*>(q) = w;
  } else {
    *reinterpret_cast<f32x4*>(q) = v;
  }
}

// Split operands.  An fp32 value x is carried as bf16 hi = RNE(x) plus
// bf16 lo = RNE(x - hi); an MFMA product with a split operand is taken as
// hi * b + lo * b, which keeps about 16 significant bits of x instead of 8.
// On the fp32 path (T = float) there is no split: lo is never formed or used.
template <typename T>
__device__ __forceinline__ void split2(float x, T& hi, T& lo) {
  hi = from_f32<T>(x);
  lo = from_f32<T>(x - to_f32(hi));
}

// store_acc_t of a split tile: hi into dh, lo into dl (dl unused for fp32)
template <typename T>
__device__ __forceinline__ void store_acc_t2(T* dh, T* dl, int ld, int r0, int c0, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 h4, l4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      T hi, lo;
      split2<T>(v[i], hi, lo);
      h4[i] = hi;
      l4[i] = lo;
    }
    const int64_t off = (int64_t)(c0 + acc_col()) * ld + r0 + acc_row0();
    *reinterpret_cast<t4*>(dh + off) = h4;
    *reinterpret_cast<t4*>(dl + off) = l4;
  } else {
    store_acc_t(dh, ld, r0, c0, v);
  }
}

// RowK fragment of the fp32 LDS matrix x(i, k) = p[i * ld + k] * sk(k),
// split into hi and lo (bf16) or taken as is (fp32).  p rows 16-byte aligned.
template <typename T, typename SK>
__device__ __forceinline__ void frag_rowk_f32(const float* p, int ld, int i0, int k0, SK&& sk,
                                              typename Mma<T>::frag& hi, typename Mma<T>::frag& lo) {
  const int l = lane_id();
  if constexpr (Mma<T>::KPL == 8) {
    const int kb = k0 + 8 * (l >> 4);
    const float* q = p + (i0 + (l & 15)) * ld + kb;
    const f32x4 a = *reinterpret_cast<const f32x4*>(q);
    const f32x4 b = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16 h, lw;
      split2<bf16>((j < 4 ? a[j] : b[j - 4]) * sk(kb + j), h, lw);
      hi[j] = h;
      lo[j] = lw;
    }
  } else {
    const int k = k0 + (l >> 4);
    hi = p[(i0 + (l & 15)) * ld + k] * sk(k);
  }
}

// ColK fragment of the 16-bit LDS matrix x(i, k) = p[k * ld + i] * sk(k),
// split into hi and lo (fp32: taken as is).
template <typename T, typename SK>
__device__ __forceinline__ void frag_colk_scaled(const T* p, int ld, int i0, int k0, SK&& sk,
                                                 typename Mma<T>::frag& hi, typename Mma<T>::frag& lo) {
  const typename Mma<T>::frag raw = frag_colk_lds(p, ld, i0, k0);
  const int l = lane_id();
  if constexpr (Mma<T>::KPL == 8) {
    const int kb = k0 + 8 * (l >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16 h, lw;
      split2<bf16>((float)raw[j] * sk(kb + j), h, lw);
      hi[j] = h;
      lo[j] = lw;
    }
  } else {
    hi = raw * sk(k0 + (l >> 4));
  }
}

// Store / load an accumulator tile in accumulator order (4 contiguous
// elements per lane: 8-byte or 16-byte accesses, 64 lanes contiguous).
template <typename T>
__device__ __forceinline__ void store_acc4(T* q, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 w = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
    *reinterpret_cast<t4*>(q) = w;
  } else {
    *reinterpret_cast<f32x4*>(q) = v;
  }
}

// store_acc4 with a non-temporal (streaming) store, for data that no other
// workgroup of the same kernel reads and that a later kernel reads once:
// it then does not displace, in L2 and the Infinity Cache, the chunk
// operands that several column tiles of a scan share.  Used for the
// per-tile terms the WY passes hand to the scans (U; scale P^T dO, scale
// Qg^T dO) and for the forward's state snapshots; the backward WY pass
// stores T the same way, and the readers of these buffers load them with
// non-temporal loads as well.  (The shared W, K^T, Q, P and W^T, K
// fragments keep ordinary stores and loads: loading them non-temporally
// made the forward scan 27 us slower.  The reverse scan's dh snapshots and
// dDelta keep ordinary stores too: the gradient kernel, which runs right
// after it, then finds them in the Infinity Cache.)
template <typename T>
__device__ __forceinline__ void store_acc4_nt(T* q, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 w = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
    __builtin_nontemporal_store(w, reinterpret_cast<t4*>(q));
  } else {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(q));
  }
}

// Store an accumulator tile in its own orientation: dst[(r0 + i) * ld + c0 + c].
template <typename T>
__device__ __forceinline__ void store_acc(T* dst, int64_t ld, int r0, int c0, f32x4 v) {
  T* q = dst + (int64_t)(r0 + acc_row0()) * ld + c0 + acc_col();
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i * ld] = from_f32<T>(v[i]);
}

// ---------------------------------------------------------------------------
// Gate factors.  The chunk-local cumulative sum gamma is formed exactly as a
// pair of floats (hi + lo, error-free two-sum additions in the wave scan).
// A factor exp(gamma_r - gamma_s) is one
// hardware 2^x (v_exp_f32) of ((hi_r - hi_s) + (lo_r - lo_s)) log2(e): the
// difference is taken before anything is rounded at the scale of gamma
// itself.  With fast decay (gamma of -100 and more at the end of a chunk) an
// fp32 cumulative sum, or gamma scaled by log2(e) before the difference,
// would put errors of ~1e-5 relative into factors near 1.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// exp(gamma_r - gamma_s) from the hi / lo arrays of gamma.  The lo part is
// used on the fp32 path only: on the bf16 path the factors enter products
// whose operands are rounded to 8 bits, so the hi difference (relative
// error ~|gamma| 2^-24) is ample and saves the extra LDS reads and VALU work.
template <bool EXACT>
__device__ __forceinline__ float gate_factor(const float* hi, const float* lo, int r, int s) {
  if constexpr (EXACT) return exp2_hw(((hi[r] - hi[s]) + (lo[r] - lo[s])) * LOG2E);
  else return exp2_hw((hi[r] - hi[s]) * LOG2E);
}

// ---------------------------------------------------------------------------
// Wavefront scans over 64 lanes.
// inclusive scan in float pairs (hi + lo): each addition's rounding error is
// recovered exactly (Knuth's two-sum) and carried in lo, so hi + lo is the
// sum to about 2^-48 relative
__device__ __forceinline__ float wave_incl_scan_2f(float x, float& lo_out) {
  const int l = lane_id();
  float hi = x, lo = 0.f;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float yh = __shfl_up(hi, d, 64), yl = __shfl_up(lo, d, 64);
    if (l >= d) {
      const float sh = hi + yh;
      const float bb = sh - hi;
      const float err = (hi - (sh - bb)) + (yh - bb);
      hi = sh;
      lo = lo + yl + err;
      const float t = hi + lo;
      lo = lo - (t - hi);
      hi = t;
    }
  }
  lo_out = lo;
  return hi;
}
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  return x;
}
// suffix sum: out_l = sum_{m >= l} x_m
__device__ __forceinline__ float wave_suffix_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_down(x, d, 64);
    if (l + d < 64) x += y;
  }
  return x;
}
// sum over the 16 lanes sharing l >> 4
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}
// sum over the 4 lane groups sharing l & 15
__device__ __forceinline__ float sum4g(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// ---------------------------------------------------------------------------
// Chunk geometry.  Chunks hold C = 64 tokens and never straddle sequences;
// the last chunk of a sequence may be partial.  Fixed-length batches use
// arithmetic; packed batches use the device chunk table built by the plan
// kernel (seq_chunk[n] = first chunk slot of sequence n, chunk_seq[c] =
// sequence of slot c or -1).
constexpr int CH = 64;

struct Geo {
  int H;
  int N;            // sequences
  int T_fixed;      // tokens per sequence (fixed-length batches)
  int nc_per_seq;   // chunks per sequence (fixed-length batches)
  int nchunks;      // chunk slots (grid size of chunk-parallel kernels)
  int T_total;      // packed batches: size of the token dimension (clamps cu_seqlens)
  const int* cu;        // packed: cu_seqlens [N+1], else nullptr
  const int* seq_chunk; // packed: [N+1]
  const int* chunk_seq; // packed: [nchunks]
  int cp;               // intra-card context-parallel segments per sequence (>= 1)
};

__device__ __forceinline__ bool chunk_lookup(const Geo& g, int ci, int& n, int& t0, int& len) {
  if (g.cu == nullptr) {
    if (g.nc_per_seq <= 0) return false;
    n = ci / g.nc_per_seq;
    const int j = ci - n * g.nc_per_seq;
    t0 = n * g.T_fixed + j * CH;
    len = min(CH, g.T_fixed - j * CH);
    return len > 0;
  }
  n = g.chunk_seq[ci];
  if (n < 0) return false;
  const int j = ci - g.seq_chunk[n];
  // cu_seqlens is clamped into [0, T_total] so that a contract violation can
  // never address tokens outside the buffers
  const int s = min(max(g.cu[n], 0), g.T_total);
  const int e = min(max(g.cu[n + 1], s), g.T_total);
  t0 = s + j * CH;
  len = min(CH, e - t0);
  return len > 0;
}

// chunk slots [c0, c0 + nc) and tokens [ts, ts + tl) of sequence n
__device__ __forceinline__ void seq_range(const Geo& g, int n, int& c0, int& nc, int& ts, int& tl) {
  if (g.cu == nullptr) {
    c0 = n * g.nc_per_seq;
    nc = g.nc_per_seq;
    ts = n * g.T_fixed;
    tl = g.T_fixed;
  } else {
    c0 = g.seq_chunk[n];
    nc = g.seq_chunk[n + 1] - c0;
    ts = min(max(g.cu[n], 0), g.T_total);
    tl = min(max(g.cu[n + 1], ts), g.T_total) - ts;
    nc = min(nc, (tl + CH - 1) / CH);
  }
}

// chunk slots [c0, c0 + nc) and tokens [ts, ts + tl) of context-parallel
// segment s of sequence n: segments hold ceil(chunks / cp) chunks each, the
// trailing ones may be short or empty
__device__ __forceinline__ void seg_range(const Geo& g, int n, int s, int& c0, int& nc, int& ts, int& tl) {
  seq_range(g, n, c0, nc, ts, tl);
  const int per = (nc + g.cp - 1) / g.cp;
  const int b = min(s * per, nc), e = min(b + per, nc);
  c0 += b;
  nc = e - b;
  ts += b * CH;
  tl = max(0, min(tl - b * CH, nc * CH));
}

// XCD-aware placement of the serial-scan workgroups.  Workgroups are handed
// to the 8 XCDs in turn (workgroup b runs on XCD b % 8), so unit p gets all
// its column tiles on XCD p % 8: the tiles read the same chunk operands and
// share them in that XCD's L2.  The grid is 8 * ceil(units / 8) * ntiles;
// returns false for the padding workgroups.
__device__ __forceinline__ bool unit_of(int b, int units, int ntiles, int& p, int& jt) {
  const int x = b & 7, k = b >> 3;
  jt = k % ntiles;
  p = (k / ntiles) * 8 + x;
  return p < units;
}

// ---------------------------------------------------------------------------
// Workgroup barrier of every kernel.  The race-test build of the library
// (compiled with GDR_DEBUG_DELAY) puts chosen waves to sleep after a
// pseudo-random subset of barriers: a wave that reads or overwrites LDS
// data another wave still needs, without a barrier in between, then sees
// different data and the results change.  The sleeps change no arithmetic,
// so that build's outputs with and without delays must be bitwise equal.
#ifdef GDR_DEBUG_DELAY
struct DelayCfg {
  int wave;    // wave to delay, -1: every wave
  int mod;     // delay after a barrier when a cycle-counter hash % mod == 0
  int iters;   // s_sleep(127) repetitions per delay; 0 turns delays off
  int salt;    // varies the pseudo-random choice between runs
};
// one copy per translation unit, written by the host before a launch
static __constant__ DelayCfg g_delay;
__device__ __forceinline__ void debug_delay() {
  const DelayCfg c = g_delay;
  if (c.iters <= 0 || c.mod <= 0) return;
  if (c.wave >= 0 && c.wave != wave_id()) return;
  const uint32_t t = (uint32_t)(__builtin_readcyclecounter() >> 6) ^ (blockIdx.x * 2654435761u) ^ (uint32_t)c.salt;
  if (t % (uint32_t)c.mod != 0) return;
  for (int i = 0; i < c.iters; ++i) __builtin_amdgcn_s_sleep(127);
}
#define GDR_SYNC()          \
  do {                      \
    __syncthreads();        \
    ::gdr::debug_delay();   \
  } while (0)
#else
#define GDR_SYNC() __syncthreads()
#endif

}  // namespace gdr
