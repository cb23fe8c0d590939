// gdr_fwd.hip -- forward kernels of the chunked gated delta rule on gfx950.
//
// The operator is the chunked gated delta rule of FlashQLA PR #34 ("SM120/121 :
// Add support for fused backward kernel", section "Summary"); the pages give
// no formula, so the kernels compute the standard gated delta recurrence
//   S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//   o_t = scale S_t q_t
// chunk-wise.  Inside a chunk of 64 rows with state h (KV form, DK x DV) at
// its start, gamma = inclusive cumsum of g, Gam[r][s] = exp(gamma_r - gamma_s)
// for s <= r, and
//   A = strictly_lower(diag(beta) K K^T * Gam),   T = (I + A)^-1
//   W = T diag(beta e^gamma) K,   U = T diag(beta) V
//   Delta = U - W h
//   O = scale (diag(e^gamma) Q h + (Q K^T * Gam) Delta)
//   h <- e^{gamma_L} h + (diag(e^{gamma_L - gamma}) K)^T Delta.
// exp(-gamma) is never formed on its own: every exponent is a difference
// gamma_r - gamma_s with s <= r, or gamma_L - gamma_r, taken after masking.
//
// Kernels (all launched on the caller's stream, no host synchronisation):
//   k_plan      packed batches: cu_seqlens -> chunk table on the device
//   k_wy        chunk-parallel: gamma, T, W, U (and backward extras)
//   k_scan_fwd  serial over chunks per (sequence, head, DV tile): the state
//               tile lives in registers (fp32 MFMA accumulators) with a bf16
//               copy in LDS; writes per-chunk snapshots, o and h_T
#include "gdr_kernels.h"

namespace gdr {

__device__ __forceinline__ int seq_len_clamped(const int* cu, int n, int T_total) {
  const int s = min(max(cu[n], 0), T_total);
  return min(max(cu[n + 1], s), T_total) - s;
}

// ---------------------------------------------------------------------------
// k_plan: one workgroup of 1024 threads builds seq_chunk[0..N] (first chunk
// slot of each sequence, exclusive scan of ceil(len/64)) and chunk_seq[c]
// (sequence of chunk slot c, -1 past the last chunk).  N <= GDR_MAX_SEQS.
__global__ __launch_bounds__(1024) void k_plan(const int* cu, int N, int T_total, int nchunks,
                                              int* seq_chunk, int* chunk_seq) {
  __shared__ int s_off[GDR_MAX_SEQS + 1];
  __shared__ int s_part[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int n0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int n = n0 + i;
    if (n < N) {
      local += (seq_len_clamped(cu, n, T_total) + CH - 1) / CH;
    }
  }
  s_part[tid] = local;
  __syncthreads();
  // inclusive Hillis-Steele scan over 1024 partials
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = (tid >= d) ? s_part[tid - d] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int run = s_part[tid] - local;
  for (int i = 0; i < per; ++i) {
    const int n = n0 + i;
    if (n < N) {
      s_off[n] = min(run, nchunks);
      run += (seq_len_clamped(cu, n, T_total) + CH - 1) / CH;
    }
  }
  if (tid == 1023) s_off[N] = min(s_part[1023], nchunks);
  __syncthreads();
  for (int n = tid; n <= N; n += 1024) seq_chunk[n] = s_off[n];
  const int total = s_off[N];
  for (int c = tid; c < nchunks; c += 1024) {
    int res = -1;
    if (c < total) {
      // last n with s_off[n] <= c (empty sequences share offsets; the last
      // one of a run of equal offsets is the non-empty owner)
      int lo = 0, hi = N;  // invariant: s_off[lo] <= c < s_off[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= c) lo = mid;
        else hi = mid;
      }
      res = lo;
    }
    chunk_seq[c] = res;
  }
}

// ---------------------------------------------------------------------------
// k_wy: per (chunk, head).  Computes gamma, A, T = (I + A)^-1 (blocked:
// 16 x 16 diagonal blocks by forward substitution, then off-diagonal block
// rows T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj on fp32 MFMA), W and U on the
// operand-type MFMA, and P = Q K^T * Gam; writes everything the scans and
// the gradient kernel consume, in fragment / accumulator order (see
// gdr_kernels.h).
template <typename T, int DK, bool BWD>
__global__ __launch_bounds__(256) void k_wy(const WyArgs a) {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P;
  constexpr int L64 = 64 + P;
  constexpr int LDF = 68;
  constexpr int DVB = dvb_of<T>();
  constexpr int LDV = DVB + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int R1 = cmax(cmax(2 * 64 * LDF * 4, (64 * LDK + 64 * LDV) * (int)sizeof(T)),
                          (64 * LDK + 64 * L64) * (int)sizeof(T));
  extern __shared__ __align__(16) char smem[];
  T* sK = (T*)smem;
  char* r1 = smem + 64 * LDK * sizeof(T);
  float* sA = (float*)r1;              // A (fp32), then dead
  float* sTm = sA + 64 * LDF;          // T (fp32), then dead
  T* sW = (T*)r1;                      // W (r, dk), after T1/T2 are built
  T* sV = sW + 64 * LDK;               // V / dO block (r, dv)
  T* sQ = (T*)r1;                      // Q (r, dk), after W and V are done
  T* sP = sQ + 64 * LDK;               // P (r, s)
  T* sT1 = (T*)(r1 + R1);
  T* sT2 = sT1 + 64 * L64;
  float* sX = (float*)(sT2 + 64 * L64);
  float* sg = sX + 4 * 16 * 20;
  float* sb = sg + 64;
  float* seg = sb + 64;
  float* sE = seg + 64;

  const int ci = blockIdx.x, h = blockIdx.y;
  int n, t0, len;
  if (!chunk_lookup(a.geo, ci, n, t0, len)) return;
  const int H = a.geo.H, DV = a.DV;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t ch = (int64_t)h * a.geo.nchunks + ci;
  const T* kp = (const T*)a.k;
  const T* vp = (const T*)a.v;

  if (w == 0) {
    float gv = 0.f, bv = 0.f;
    if (l < len) {
      gv = a.g[(int64_t)(t0 + l) * H + h];
      bv = a.beta[(int64_t)(t0 + l) * H + h];
    }
    const float gm = wave_incl_scan(gv);
    const float gL = __shfl(gm, 63, 64);
    const float eg = expf(gm), eE = expf(gL - gm);
    sg[l] = gm;
    sb[l] = bv;
    seg[l] = eg;
    sE[l] = eE;
    a.gam[ch * GSTRIDE + l] = gm;
    a.gam[ch * GSTRIDE + 64 + l] = eg;
    a.gam[ch * GSTRIDE + 128 + l] = eE;
  }
  load_rows<T, DK>(sK, LDK, kp + ((int64_t)t0 * H + h) * DK, (int64_t)H * DK, len);
  __syncthreads();

  // A = strictly_lower(diag(beta) K K^T * Gam): rows 16w, 4 column tiles
  {
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = frag_rowk(sK, LDK, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sK, LDK, 16 * nt, ks), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + acc_row0() + i, s = 16 * nt + acc_col();
        sA[r * LDF + s] = (s < r) ? sb[r] * acc[nt][i] * expf(sg[r] - sg[s]) : 0.f;
      }
  }
  __syncthreads();

  // diagonal 16 x 16 blocks of T by forward substitution (wave 0: lane =
  // (block, column)); strictly-upper blocks are zero
  if (w == 0) {
    const int b = l >> 4, c = l & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= sA[(16 * b + i) * LDF + 16 * b + j] * x[j];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sTm[(16 * b + i) * LDF + 16 * b + c] = x[i];
  }
  for (int e = tid; e < 64 * 64; e += 256) {
    const int r = e >> 6, s = e & 63;
    if ((s >> 4) > (r >> 4)) sTm[r * LDF + s] = 0.f;
  }
  __syncthreads();
  // off-diagonal block rows (fp32 MFMA, k = 4 per instruction)
  for (int bi = 1; bi < 4; ++bi) {
    if (w < bi) {
      f32x4 X = zero4();
      for (int kb = w; kb < bi; ++kb)
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4) {
          const float af = sA[(16 * bi + (l & 15)) * LDF + 16 * kb + kk + (l >> 4)];
          const float bf = sTm[(16 * kb + kk + (l >> 4)) * LDF + 16 * w + (l & 15)];
          X = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bf, X, 0, 0, 0);
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) sX[w * 320 + (acc_row0() + i) * 20 + acc_col()] = X[i];
    }
    __syncthreads();
    if (w < bi) {
      f32x4 Y = zero4();
#pragma unroll
      for (int kk = 0; kk < 16; kk += 4) {
        const float af = sTm[(16 * bi + (l & 15)) * LDF + 16 * bi + kk + (l >> 4)];
        const float bf = sX[w * 320 + (kk + (l >> 4)) * 20 + (l & 15)];
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bf, Y, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sTm[(16 * bi + acc_row0() + i) * LDF + 16 * w + acc_col()] = -Y[i];
    }
    __syncthreads();
  }

  // T1 = T diag(beta e^gamma), T2 = T diag(beta) in the operand type
  for (int e = tid; e < 64 * 64; e += 256) {
    const int r = e >> 6, s = e & 63;
    const float t = sTm[r * LDF + s];
    sT1[r * L64 + s] = from_f32<T>(t * sb[s] * seg[s]);
    sT2[r * L64 + s] = from_f32<T>(t * sb[s]);
    if constexpr (BWD) a.Tm[ch * 4096 + e] = t;
  }
  __syncthreads();  // sA / sTm are dead from here

  // W^T = K^T T1^T (DK x 64): wave w owns dk rows [w DK/4, (w+1) DK/4);
  // staged row-major in LDS, then written out in fragment order
  {
    constexpr int MT = DK / 64;
    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      typename Mma<T>::frag af[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) af[mt] = frag_colk_lds(sK, LDK, w * (DK / 4) + 16 * mt, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const auto bf = frag_rowk(sT1, L64, 16 * nt, ks);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = Mma<T>::mma(af[mt], bf, acc[mt][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) store_acc_t(sW, LDK, w * (DK / 4) + 16 * mt, 16 * nt, acc[mt][nt]);
  }
  __syncthreads();
  write_afrag<T, 64, DK>((T*)a.Wf + ch * 64 * DK, [&](int i, int k) { return to_f32(sW[i * LDK + k]); });
  if constexpr (BWD) {
    write_afrag<T, DK, 64>((T*)a.WTf + ch * DK * 64, [&](int i, int k) { return to_f32(sW[k * LDK + i]); });
    write_afrag<T, 64, DK>((T*)a.Ktf + ch * 64 * DK, [&](int i, int k) { return sE[i] * to_f32(sK[i * LDK + k]); });
  }
  if (a.KtTf)
    write_afrag<T, DK, 64>((T*)a.KtTf + ch * DK * 64, [&](int i, int k) { return sE[k] * to_f32(sK[k * LDK + i]); });

  // U = T2 V per DV block (rows 16w), written in accumulator order
  for (int dv0 = 0; dv0 < DV; dv0 += DVB) {
    __syncthreads();
    load_rows<T, DVB>(sV, LDV, vp + ((int64_t)t0 * H + h) * DV + dv0, (int64_t)H * DV, len);
    __syncthreads();
    f32x4 acc[DVB / 16];
#pragma unroll
    for (int nt = 0; nt < DVB / 16; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const auto af = frag_rowk(sT2, L64, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt)
        acc[nt] = Mma<T>::mma(af, frag_colk_lds(sV, LDV, 16 * nt, ks), acc[nt]);
    }
    T* Ub = (T*)a.Ua + ch * 64 * DV;
#pragma unroll
    for (int nt = 0; nt < DVB / 16; ++nt) store_acc4(Ub + acc_off(w, dv0 / 16 + nt, DV), acc[nt]);
  }
  if constexpr (BWD) {
    // dO^T in fragment order, per DV block
    const T* dop = (const T*)a.dO;
    for (int dv0 = 0; dv0 < DV; dv0 += DVB) {
      __syncthreads();
      load_rows<T, DVB>(sV, LDV, dop + ((int64_t)t0 * H + h) * DV + dv0, (int64_t)H * DV, len);
      __syncthreads();
      write_afrag<T, DVB, 64>((T*)a.dOf + ch * DV * 64 + (int64_t)dv0 * 64,
                              [&](int i, int k) { return to_f32(sV[k * LDV + i]); });
    }
  }

  __syncthreads();  // sW / sV are dead from here
  load_rows<T, DK>(sQ, LDK, (const T*)a.q + ((int64_t)t0 * H + h) * DK, (int64_t)H * DK, len);
  __syncthreads();
  // P = Q K^T * Gam (diagonal included), computed as P^T (rows s = 16w),
  // staged row-major (r, s) in LDS
  {
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = frag_rowk(sK, LDK, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sQ, LDK, 16 * nt, ks), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * w + acc_row0() + i, r = 16 * nt + acc_col();
        acc[nt][i] = (s <= r) ? acc[nt][i] * expf(sg[r] - sg[s]) : 0.f;
      }
      store_acc_t(sP, L64, 16 * w, 16 * nt, acc[nt]);
    }
  }
  __syncthreads();
  if constexpr (!BWD) {
    write_afrag<T, 64, 64>((T*)a.Pf + ch * 4096, [&](int i, int k) { return to_f32(sP[i * L64 + k]); });
    write_afrag<T, 64, DK>((T*)a.Qgf + ch * 64 * DK, [&](int i, int k) { return seg[i] * to_f32(sQ[i * LDK + k]); });
  } else {
    const float sc = a.scale;
    write_afrag<T, 64, 64>((T*)a.PsTf + ch * 4096, [&](int i, int k) { return sc * to_f32(sP[k * L64 + i]); });
    write_afrag<T, DK, 64>((T*)a.QgsTf + ch * DK * 64,
                           [&](int i, int k) { return sc * seg[k] * to_f32(sQ[k * LDK + i]); });
  }
}

// ---------------------------------------------------------------------------
// k_scan_fwd: per (sequence, head, DV tile).  Serial over the sequence's
// chunks.  The state tile h (DK x DVT, fp32) is held in MFMA accumulators
// (wave w owns dk rows [w DK/4, (w+1) DK/4)); a bf16 copy h^T lives in LDS
// as the B operand of W h (and of Q h for the output).  Delta^T goes to LDS
// as the B operand of the update h <- e^{gamma_L} h + Kt^T Delta and of
// P Delta.  All per-chunk operands that do not depend on h (W, Kt^T, U, Q,
// P, the gate exponentials) are loaded raw into a ring of SCAN_STAGES
// register sets, SCAN_STAGES - 1 chunks ahead; nothing touches a loaded
// value before its chunk is processed, so the loads stay in flight while
// earlier chunks run.  With OUT the kernel also writes
// o = scale (e^gamma Q h + P Delta).
#define SCAN_STAGES 3

template <typename T, typename HS, int DK, int DVT, bool OUT>
__global__ __launch_bounds__(256) void k_scan_fwd(const ScanFwdArgs a) {
  constexpr int P = pad_of<T>();
  constexpr int LDH = DK + P;
  constexpr int LDD = 64 + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int KS = DK / KW;
  constexpr int KS64 = 64 / KW;
  constexpr int MTH = DK / 64;
  constexpr int NT = DVT / 16;
  constexpr int S = sizeof(T) == 2 ? SCAN_STAGES : 2;  // fp32 fragments are 8x larger
  typedef typename Mma<T>::frag frag;
  typedef T t4 __attribute__((ext_vector_type(4)));
  constexpr int LDO = DVT + P;
  __shared__ __align__(16) T sH[DVT * LDH];
  __shared__ __align__(16) T sD[DVT * LDD];
  __shared__ __align__(16) T sO[OUT ? 64 * LDO : 1];  // output staging (each wave: its rows)

  const int H = a.geo.H, DV = a.DV;
  const int Pn = a.geo.N * H;
  const int b = blockIdx.x;
  const int jt = b / Pn, p = b - jt * Pn;
  const int n = p / H, h = p - n * H;
  const int dv0 = jt * DVT;
  int c0, nc, ts, tl;
  seq_range(a.geo, n, c0, nc, ts, tl);
  const int w = wave_id();
  const int l = lane_id();
  const int dkw = w * (DK / 4);
  const int rw = 16 * w;
  const int64_t chb = (int64_t)h * a.geo.nchunks + c0;   // chunk-head index of chunk 0

  f32x4 acc_h[MTH][NT];
  const int64_t sb = (int64_t)(n * H + h) * DK * DV;
#pragma unroll
  for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = dkw + 16 * mt + acc_row0() + i, dv = dv0 + 16 * nt + acc_col();
        float v = 0.f;
        if (a.h0) v = (a.layout == 0) ? a.h0[sb + (int64_t)dk * DV + dv] : a.h0[sb + (int64_t)dv * DK + dk];
        acc_h[mt][nt][i] = v;
      }
#pragma unroll
  for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) store_acc_t(sH, LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);

  struct Ops {
    frag wf[KS];           // W rows 16w
    frag kf[MTH][KS64];    // Kt^T rows dkw.., k = chunk row
    t4 u[NT];              // U (accumulator order, raw)
    frag qf[KS];           // e^gamma Q rows 16w
    frag pf[KS64];         // P rows 16w
    float eL;              // e^{gamma_L}
  };
  auto load_ops = [&](int c, Ops& o) {
    const int64_t ch = chb + c;
    const T* Wb = (const T*)a.Wf + ch * 64 * DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) o.wf[ks] = frag_af<T, DK>(Wb, w, ks);
    const T* Kb = (const T*)a.KtTf + ch * DK * 64;
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS64; ++ks) o.kf[mt][ks] = frag_af<T, 64>(Kb, dkw / 16 + mt, ks);
    const T* Ub = (const T*)a.Ua + ch * 64 * DV;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o.u[nt] = *reinterpret_cast<const t4*>(Ub + acc_off(w, dv0 / 16 + nt, DV));
    o.eL = a.gam[ch * GSTRIDE + 64 + 63];
    if constexpr (OUT) {
      const T* Qb = (const T*)a.Qgf + ch * 64 * DK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o.qf[ks] = frag_af<T, DK>(Qb, w, ks);
      const T* Pb = (const T*)a.Pf + ch * 4096;
#pragma unroll
      for (int ks = 0; ks < KS64; ++ks) o.pf[ks] = frag_af<T, 64>(Pb, w, ks);
    }
  };

  auto process = [&](int c, Ops& o) {
    const int64_t ch = chb + c;
    {
      HS* hb = (HS*)a.hs + ch * DK * DV;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) store_acc4(hb + acc_off(dkw / 16 + mt, dv0 / 16 + nt, DV), acc_h[mt][nt]);
    }
    __syncthreads();  // h^T in LDS is complete; last chunk's readers of Delta^T are done
    // W h and (with OUT) Q h, rows 16w
    f32x4 acc_d[NT], acc_o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc_d[nt] = acc_o[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const frag bh = frag_rowk(sH, LDH, 16 * nt, ks * KW);
        acc_d[nt] = Mma<T>::mma(o.wf[ks], bh, acc_d[nt]);
        if constexpr (OUT) acc_o[nt] = Mma<T>::mma(o.qf[ks], bh, acc_o[nt]);
      }
    // Delta = U - W h
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_d[nt][i] = to_f32(o.u[nt][i]) - acc_d[nt][i];
      store_acc_t(sD, LDD, rw, 16 * nt, acc_d[nt]);
    }
    __syncthreads();  // Delta^T complete; all readers of h^T are done
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_h[mt][nt] *= o.eL;
#pragma unroll
    for (int ks = 0; ks < KS64; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const frag bd = frag_rowk(sD, LDD, 16 * nt, ks * KW);
        if constexpr (OUT) acc_o[nt] = Mma<T>::mma(o.pf[ks], bd, acc_o[nt]);
#pragma unroll
        for (int mt = 0; mt < MTH; ++mt) acc_h[mt][nt] = Mma<T>::mma(o.kf[mt][ks], bd, acc_h[mt][nt]);
      }
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_acc_t(sH, LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);
    if constexpr (OUT) {
      // each wave stages its 16 output rows in LDS and writes them back as
      // 16-byte pieces (LDS accesses of one wave are ordered: no barrier)
      const int t0 = ts + c * CH;
      const int len = min(CH, tl - c * CH);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_acc(sO, LDO, rw, 16 * nt, a.scale * acc_o[nt]);
      constexpr int VE = 16 / sizeof(T);
      constexpr int PPR = DVT / VE;  // 16-byte pieces per row
      typedef float f4 __attribute__((ext_vector_type(4)));
      T* op = (T*)a.o + ((int64_t)t0 * H + h) * DV + dv0;
      // compile-time trip count: keeps the count of memory operations
      // static, so the prefetched loads stay in flight across chunks
#pragma unroll
      for (int it = 0; it < (16 * PPR + 63) / 64; ++it) {
        const int pc = l + 64 * it;
        const int r = rw + pc / PPR, cc = (pc % PPR) * VE;
        if (pc < 16 * PPR && r < len)
          *reinterpret_cast<f4*>(op + (int64_t)r * H * DV + cc) = *reinterpret_cast<const f4*>(sO + r * LDO + cc);
      }
    }
  };

  // Chunk c lives in register stage c % S.  The main loop handles S chunks
  // per trip with unconditional prefetches (the index is clamped to the last
  // chunk, so the tail re-reads it): the number of memory operations between
  // a prefetch and its use is then fixed, and the compiler's wait counts let
  // the prefetched loads stay in flight.  A static tail runs the last
  // nc % S chunks.
  if (nc > 0) {
    Ops st[S];
#pragma unroll
    for (int s = 0; s < S - 1; ++s) load_ops(min(s, nc - 1), st[s]);
    int cb = 0;
    for (; cb + S <= nc; cb += S) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        load_ops(min(cb + s + S - 1, nc - 1), st[(s + S - 1) % S]);
        process(cb + s, st[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (cb + s < nc) process(cb + s, st[s]);
  }
  if (a.hT) {
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = dkw + 16 * mt + acc_row0() + i, dv = dv0 + 16 * nt + acc_col();
          if (a.layout == 0) a.hT[sb + (int64_t)dk * DV + dv] = acc_h[mt][nt][i];
          else a.hT[sb + (int64_t)dv * DK + dk] = acc_h[mt][nt][i];
        }
  }
}

// ---------------------------------------------------------------------------
// host-side launchers

template <typename T, int DK, bool BWD>
static size_t wy_smem() {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P, L64 = 64 + P, LDF = 68, DVB = dvb_of<T>(), LDV = DVB + P;
  constexpr int R1 = cmax(cmax(2 * 64 * LDF * 4, (64 * LDK + 64 * LDV) * (int)sizeof(T)),
                          (64 * LDK + 64 * L64) * (int)sizeof(T));
  return 64 * LDK * sizeof(T) + R1 + 2 * 64 * L64 * sizeof(T) + 4 * 16 * 20 * 4 + 4 * 64 * 4;
}

template <typename T, int DK, bool BWD>
static hipError_t launch_wy_t(const WyArgs& a, hipStream_t st) {
  const size_t sm = wy_smem<T, DK, BWD>();
  hipError_t e = hipFuncSetAttribute((const void*)k_wy<T, DK, BWD>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_wy<T, DK, BWD>), dim3(a.geo.nchunks, a.geo.H), dim3(256), sm, st, a);
  return hipGetLastError();
}

hipError_t launch_plan(const int* cu, int N, int T_total, int nchunks, int* seq_chunk, int* chunk_seq,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, cu, N, T_total, nchunks, seq_chunk, chunk_seq);
  return hipGetLastError();
}

hipError_t launch_wy(const WyArgs& a, bool f32, int DK, bool bwd, hipStream_t st) {
  if (f32) {
    if (DK == 64) return bwd ? launch_wy_t<float, 64, true>(a, st) : launch_wy_t<float, 64, false>(a, st);
    return bwd ? launch_wy_t<float, 128, true>(a, st) : launch_wy_t<float, 128, false>(a, st);
  }
  if (DK == 64) return bwd ? launch_wy_t<bf16, 64, true>(a, st) : launch_wy_t<bf16, 64, false>(a, st);
  return bwd ? launch_wy_t<bf16, 128, true>(a, st) : launch_wy_t<bf16, 128, false>(a, st);
}

template <typename T, typename HS, int DK, bool OUT>
static hipError_t launch_scan_fwd_t(const ScanFwdArgs& a, int dvt, hipStream_t st) {
  const int Pn = a.geo.N * a.geo.H;
  const int grid = Pn * (a.DV / dvt);
  if (grid == 0) return hipSuccess;
  if (dvt == 16) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 16, OUT>), dim3(grid), dim3(256), 0, st, a);
  else if (dvt == 32) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 32, OUT>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 64, OUT>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, typename HS>
static hipError_t launch_scan_fwd_d(const ScanFwdArgs& a, int DK, int dvt, hipStream_t st) {
  const bool out = a.o != nullptr;
  if (DK == 64) return out ? launch_scan_fwd_t<T, HS, 64, true>(a, dvt, st) : launch_scan_fwd_t<T, HS, 64, false>(a, dvt, st);
  return out ? launch_scan_fwd_t<T, HS, 128, true>(a, dvt, st) : launch_scan_fwd_t<T, HS, 128, false>(a, dvt, st);
}

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool f32, int hs_dtype, int DK, int dvt, hipStream_t st) {
  if (f32) return launch_scan_fwd_d<float, float>(a, DK, dvt, st);
  if (hs_dtype == GDR_F32) return launch_scan_fwd_d<bf16, float>(a, DK, dvt, st);
  if (hs_dtype == GDR_F16) return launch_scan_fwd_d<bf16, f16>(a, DK, dvt, st);
  return launch_scan_fwd_d<bf16, bf16>(a, DK, dvt, st);
}

}  // namespace gdr
