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
//               copy in LDS; writes per-chunk snapshots, Delta and h_T
//   k_out       chunk-parallel: O
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
// rows T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj on fp32 MFMA), then W and U on
// the operand-type MFMA.  Workspace outputs (chunk-major, [slot][head][..]):
//   gam [64] fp32, W [64][DK], KtT [DK][64] = (diag(e^{gL-g}) K)^T,
//   UT [DV][64] = U^T; with BWD also Tm [64][64] fp32, WT [DK][64],
//   PsT [64][64] = (scale (Q K^T * Gam))^T, QgsT [DK][64] = (scale e^g Q)^T.
template <typename T, int DK, bool BWD>
__global__ __launch_bounds__(256) void k_wy(const WyArgs a) {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P;
  constexpr int L64 = 64 + P;
  constexpr int LDF = 68;
  constexpr int DVB = dvb_of<T>();
  constexpr int LDV = DVB + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int UNION = cmax(cmax(64 * LDF * 4, 64 * LDV * (int)sizeof(T)),
                             BWD ? 64 * LDK * (int)sizeof(T) : 0);
  extern __shared__ __align__(16) char smem[];
  T* sK = (T*)smem;
  char* uni = smem + 64 * LDK * sizeof(T);
  float* sA = (float*)uni;
  float* sTm = (float*)(uni + UNION);
  T* sT1 = (T*)(sTm + 64 * LDF);
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
  const int64_t ch = (int64_t)ci * H + h;
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
    sg[l] = gm;
    sb[l] = bv;
    seg[l] = expf(gm);
    sE[l] = expf(gL - gm);
    a.gam[ch * 64 + l] = gm;
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
  __syncthreads();

  // W^T = K^T T1^T (DK x 64): wave w owns dk rows [w DK/4, (w+1) DK/4)
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
    T* Wb = (T*)a.W + ch * 64 * DK;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        store_acc_t(Wb, DK, w * (DK / 4) + 16 * mt, 16 * nt, acc[mt][nt]);
        if constexpr (BWD) store_acc((T*)a.WT + ch * DK * 64, 64, w * (DK / 4) + 16 * mt, 16 * nt, acc[mt][nt]);
      }
  }
  // KtT[dk][r] = e^{gamma_L - gamma_r} K[r][dk]
  {
    T* Kb = (T*)a.KtT + ch * DK * 64;
    for (int e = tid; e < DK * 8; e += 256) {
      const int dk = e >> 3, r0 = (e & 7) * 8;
      float vals[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) vals[j] = sE[r0 + j] * to_f32(sK[(r0 + j) * LDK + dk]);
      store8<T>(Kb + dk * 64 + r0, vals);
    }
  }

  // U^T per DV block: U = T2 V, rows 16w
  T* sV = (T*)uni;
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
    T* Ub = (T*)a.UT + (ch * DV + dv0) * 64;
#pragma unroll
    for (int nt = 0; nt < DVB / 16; ++nt) store_acc_t(Ub, 64, 16 * w, 16 * nt, acc[nt]);
  }

  if constexpr (BWD) {
    __syncthreads();
    T* sQ = (T*)uni;
    load_rows<T, DK>(sQ, LDK, (const T*)a.q + ((int64_t)t0 * H + h) * DK, (int64_t)H * DK, len);
    __syncthreads();
    // scale (Q K^T * Gam), rows r = 16w; stored transposed
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = frag_rowk(sQ, LDK, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sK, LDK, 16 * nt, ks), acc[nt]);
    }
    T* Pb = (T*)a.PsT + ch * 4096;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + acc_row0() + i, s = 16 * nt + acc_col();
        acc[nt][i] = (s <= r) ? a.scale * acc[nt][i] * expf(sg[r] - sg[s]) : 0.f;
      }
      store_acc_t(Pb, 64, 16 * w, 16 * nt, acc[nt]);
    }
    T* Qb = (T*)a.QgsT + ch * DK * 64;
    for (int e = tid; e < DK * 8; e += 256) {
      const int dk = e >> 3, r0 = (e & 7) * 8;
      float vals[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) vals[j] = a.scale * seg[r0 + j] * to_f32(sQ[(r0 + j) * LDK + dk]);
      store8<T>(Qb + dk * 64 + r0, vals);
    }
  }
}

// ---------------------------------------------------------------------------
// k_scan_fwd: per (sequence, head, DV tile).  Serial over the sequence's
// chunks.  The state tile h (DK x DVT, fp32) is held in MFMA accumulators
// (wave w owns dk rows [w DK/4, (w+1) DK/4)); a bf16 copy h^T lives in LDS
// as the B operand of Delta = U - W h.  Delta^T goes to LDS as the B operand
// of the update h <- e^{gamma_L} h + Kt^T Delta.  W and Kt^T fragments are
// read straight from the workspace into registers.
template <typename T, typename HS, int DK, int DVT>
__global__ __launch_bounds__(256) void k_scan_fwd(const ScanFwdArgs a) {
  constexpr int P = pad_of<T>();
  constexpr int LDH = DK + P;
  constexpr int LDD = 64 + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int MTH = DK / 64;
  constexpr int NT = DVT / 16;
  __shared__ __align__(16) T sH[DVT * LDH];
  __shared__ __align__(16) T sD[DVT * LDD];

  const int H = a.geo.H, DV = a.DV;
  const int Pn = a.geo.N * H;
  const int b = blockIdx.x;
  const int jt = b / Pn, p = b - jt * Pn;
  const int n = p / H, h = p - n * H;
  const int dv0 = jt * DVT;
  int c0, nc, ts, tl;
  seq_range(a.geo, n, c0, nc, ts, tl);
  const int w = wave_id();
  const int dkw = w * (DK / 4);

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

  for (int c = 0; c < nc; ++c) {
    const int64_t ch = (int64_t)(c0 + c) * H + h;
    if (a.hs) {
      HS* hb = (HS*)a.hs + (ch * DV + dv0) * DK;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) store_acc_t(hb, DK, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);
    }
    __syncthreads();
    // Delta = U - W h for rows 16w
    f32x4 acc_d[NT];
    const T* UTb = (const T*)a.UT + (ch * DV + dv0) * 64;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc_d[nt] = load4f(UTb + (16 * nt + acc_col()) * 64 + 16 * w + acc_row0());
    const T* Wb = (const T*)a.W + ch * 64 * DK;
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = Mma<T>::neg(frag_rowk(Wb, DK, 16 * w, ks));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_d[nt] = Mma<T>::mma(af, frag_rowk(sH, LDH, 16 * nt, ks), acc_d[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) store_acc_t(sD, LDD, 16 * w, 16 * nt, acc_d[nt]);
    if (a.Dt) {
      T* Db = (T*)a.Dt + (ch * DV + dv0) * 64;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_acc_t(Db, 64, 16 * w, 16 * nt, acc_d[nt]);
    }
    __syncthreads();
    const float eL = expf(a.gam[ch * 64 + 63]);
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_h[mt][nt] *= eL;
    const T* Kb = (const T*)a.KtT + ch * DK * 64;
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      typename Mma<T>::frag af[MTH];
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt) af[mt] = frag_rowk(Kb, 64, dkw + 16 * mt, ks);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const auto bf = frag_rowk(sD, LDD, 16 * nt, ks);
#pragma unroll
        for (int mt = 0; mt < MTH; ++mt) acc_h[mt][nt] = Mma<T>::mma(af[mt], bf, acc_h[mt][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_acc_t(sH, LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);
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
// k_out: per (chunk, head).  O = scale (diag(e^gamma) Q h + P Delta) with
// P = Q K^T * Gam (diagonal included); DV in blocks of DVB.
template <typename T, typename HS, int DK>
__global__ __launch_bounds__(256) void k_out(const OutArgs a) {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P;
  constexpr int L64 = 64 + P;
  constexpr int DVB = dvb_of<T>();
  constexpr int KW = Mma<T>::KW;
  extern __shared__ __align__(16) char smem[];
  T* sQ = (T*)smem;
  T* sK = sQ + 64 * LDK;
  T* sPT = sK + 64 * LDK;
  T* sH = sPT + 64 * L64;
  T* sD = sH + DVB * LDK;
  float* sg = (float*)(sD + DVB * L64);

  const int ci = blockIdx.x, h = blockIdx.y;
  int n, t0, len;
  if (!chunk_lookup(a.geo, ci, n, t0, len)) return;
  const int H = a.geo.H, DV = a.DV;
  const int tid = threadIdx.x, w = wave_id();
  const int64_t ch = (int64_t)ci * H + h;
  if (tid < 64) sg[tid] = a.gam[ch * 64 + tid];
  load_rows<T, DK>(sQ, LDK, (const T*)a.q + ((int64_t)t0 * H + h) * DK, (int64_t)H * DK, len);
  load_rows<T, DK>(sK, LDK, (const T*)a.k + ((int64_t)t0 * H + h) * DK, (int64_t)H * DK, len);
  __syncthreads();
  {
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = frag_rowk(sQ, LDK, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sK, LDK, 16 * nt, ks), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + acc_row0() + i, s = 16 * nt + acc_col();
        acc[nt][i] = (s <= r) ? acc[nt][i] * expf(sg[r] - sg[s]) : 0.f;
      }
      store_acc_t(sPT, L64, 16 * w, 16 * nt, acc[nt]);
    }
  }
  float eg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) eg[i] = expf(sg[16 * w + acc_row0() + i]);
  T* op = (T*)a.o;
  for (int dvb = 0; dvb < DV; dvb += DVB) {
    __syncthreads();
    load_rows_conv<HS, T, DK, DVB>(sH, LDK, (const HS*)a.hs + (ch * DV + dvb) * DK, DK, DVB);
    load_rows<T, 64, DVB>(sD, L64, (const T*)a.Dt + (ch * DV + dvb) * 64, 64, DVB);
    __syncthreads();
    f32x4 acc[DVB / 16];
#pragma unroll
    for (int nt = 0; nt < DVB / 16; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = frag_rowk(sQ, LDK, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sH, LDK, 16 * nt, ks), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < DVB / 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nt][i] *= eg[i];
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const auto af = frag_colk_lds(sPT, L64, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sD, L64, 16 * nt, ks), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < DVB / 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + acc_row0() + i;
        if (r < len) op[((int64_t)(t0 + r) * H + h) * DV + dvb + 16 * nt + acc_col()] = from_f32<T>(a.scale * acc[nt][i]);
      }
  }
}

// ---------------------------------------------------------------------------
// host-side launchers

template <typename T, int DK, bool BWD>
static size_t wy_smem() {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P, L64 = 64 + P, LDF = 68, DVB = dvb_of<T>(), LDV = DVB + P;
  constexpr int UNION = cmax(cmax(64 * LDF * 4, 64 * LDV * (int)sizeof(T)), BWD ? 64 * LDK * (int)sizeof(T) : 0);
  return 64 * LDK * sizeof(T) + UNION + 64 * LDF * 4 + 2 * 64 * L64 * sizeof(T) + 4 * 16 * 20 * 4 + 4 * 64 * 4;
}
template <typename T, int DK>
static size_t out_smem() {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P, L64 = 64 + P, DVB = dvb_of<T>();
  return (2 * 64 * LDK + 64 * L64 + DVB * LDK + DVB * L64) * sizeof(T) + 64 * 4;
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

template <typename T, typename HS, int DK>
static hipError_t launch_scan_fwd_t(const ScanFwdArgs& a, int dvt, hipStream_t st) {
  const int Pn = a.geo.N * a.geo.H;
  const int grid = Pn * (a.DV / dvt);
  if (grid == 0) return hipSuccess;
  if (dvt == 16) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 16>), dim3(grid), dim3(256), 0, st, a);
  else if (dvt == 32) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 32>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 64>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool f32, int hs_dtype, int DK, int dvt, hipStream_t st) {
  if (f32) return DK == 64 ? launch_scan_fwd_t<float, float, 64>(a, dvt, st) : launch_scan_fwd_t<float, float, 128>(a, dvt, st);
  if (hs_dtype == GDR_F32)
    return DK == 64 ? launch_scan_fwd_t<bf16, float, 64>(a, dvt, st) : launch_scan_fwd_t<bf16, float, 128>(a, dvt, st);
  if (hs_dtype == GDR_F16)
    return DK == 64 ? launch_scan_fwd_t<bf16, f16, 64>(a, dvt, st) : launch_scan_fwd_t<bf16, f16, 128>(a, dvt, st);
  return DK == 64 ? launch_scan_fwd_t<bf16, bf16, 64>(a, dvt, st) : launch_scan_fwd_t<bf16, bf16, 128>(a, dvt, st);
}

template <typename T, typename HS, int DK>
static hipError_t launch_out_t(const OutArgs& a, hipStream_t st) {
  const size_t sm = out_smem<T, DK>();
  hipError_t e = hipFuncSetAttribute((const void*)k_out<T, HS, DK>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_out<T, HS, DK>), dim3(a.geo.nchunks, a.geo.H), dim3(256), sm, st, a);
  return hipGetLastError();
}

hipError_t launch_out(const OutArgs& a, bool f32, int hs_dtype, int DK, hipStream_t st) {
  if (f32) return DK == 64 ? launch_out_t<float, float, 64>(a, st) : launch_out_t<float, float, 128>(a, st);
  if (hs_dtype == GDR_F32) return DK == 64 ? launch_out_t<bf16, float, 64>(a, st) : launch_out_t<bf16, float, 128>(a, st);
  if (hs_dtype == GDR_F16) return DK == 64 ? launch_out_t<bf16, f16, 64>(a, st) : launch_out_t<bf16, f16, 128>(a, st);
  return DK == 64 ? launch_out_t<bf16, bf16, 64>(a, st) : launch_out_t<bf16, bf16, 128>(a, st);
}

}  // namespace gdr
