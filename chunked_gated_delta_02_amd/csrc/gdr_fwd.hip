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
#include <climits>

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
  GDR_SYNC();
  // inclusive Hillis-Steele scan over 1024 partials
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = (tid >= d) ? s_part[tid - d] : 0;
    GDR_SYNC();
    s_part[tid] += v;
    GDR_SYNC();
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
  GDR_SYNC();
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
// operand-type MFMA with T (fp32 in LDS) taken as a split operand, and
// P = Q K^T * Gam; writes everything the scans and the gradient kernel
// consume, in fragment / accumulator order (see gdr_kernels.h).
//   forward:  W, U (fp32), K^T, Q, P (hi + lo)
//   backward: W, U, T, W^T, K, scale P^T dO and scale (e^gamma Q)^T dO (fp32)
//             (+ K^T when the forward states are recomputed)
// LDS (three tiles, so that three workgroups share a compute unit at DK = 128):
//   R0 = K (r, dk); backward: then the dO blocks, once P^T is formed
//   R1 = A (fp32), turned into T in place; then P (forward) or P^T (backward)
//   R2 = the off-diagonal scratch of T; then W staging; then the V blocks of
//        U; then Q
// and the gate vectors.
template <typename T, int DK, bool BWD>
__global__ __launch_bounds__(256) void k_wy(const WyArgs a) {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P;
  constexpr int LDF = 68;   // fp32 64-wide tiles (16-byte aligned rows)
  constexpr int DVB = dvb_of<T>();
  constexpr int LDV = DVB + P;
  constexpr int KW = Mma<T>::KW;
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int R0 = 64 * LDK * (int)sizeof(T);
  constexpr int R1 = 64 * LDF * 4;
  constexpr int R2 = cmax(64 * LDK * (int)sizeof(T), cmax(64 * LDV * (int)sizeof(T), 4 * 16 * 20 * 4));
  static_assert(64 * LDV <= 64 * LDK, "the dO blocks reuse the K tile");
  typedef typename Mma<T>::frag frag;
  extern __shared__ __align__(16) char smem[];
  T* sK = (T*)smem;
  float* sA = (float*)(smem + R0);        // A (fp32), overwritten by T
  float* sTm = sA;                        // T (fp32), until U is done
  float* sPT = sA;                        // then P (r, s) (forward) or P^T (s, r) (backward), fp32
  char* r2 = smem + R0 + R1;
  float* sX = (float*)r2;                 // off-diagonal blocks of T in the making
  T* sW = (T*)r2;                         // W (r, dk) staging
  T* sVu = (T*)r2;                        // V block (r, dv) of U
  T* sQ = (T*)r2;                         // Q (r, dk)
  T* sVd = sK;                            // dO block (r, dv) (backward, after P^T)
  float* sg = (float*)(r2 + R2);          // gamma (hi)
  float* sb = sg + 64;
  float* seg = sb + 64;
  float* sE = seg + 64;
  float* sgl = sE + 64;                   // gamma (lo)

  const int ci = blockIdx.x, h = blockIdx.y;
  int n, t0, len;
  if (!chunk_lookup(a.geo, ci, n, t0, len)) return;
  const int H = a.geo.H, DV = a.DV;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t ch = (int64_t)h * a.geo.nchunks + ci;
  const T* kp = (const T*)a.k;
  const T* vp = (const T*)a.v;
  const int64_t rowq = (int64_t)t0 * H + h;   // token-row index of chunk row 0

  // every input load is issued before the first wait (the gates by wave 0,
  // then the K, Q and first V rows), so their latencies overlap; Q and V stay
  // in registers until they are stored to LDS where needed
  float gv = 0.f, bv = 0.f;
  if (w == 0 && l < len) {
    gv = a.g[(int64_t)(t0 + l) * H + h];
    bv = a.beta[(int64_t)(t0 + l) * H + h];
  }
  RowBuf<T, DK> kbuf;
  kbuf.load(kp + rowq * DK, (int64_t)H * DK, len);
  RowBuf<T, DK> qbuf;
  RowBuf<T, DVB> vbuf;
  qbuf.load((const T*)a.q + rowq * DK, (int64_t)H * DK, len);
  // first V block for U, or (backward without U) the first dO block
  vbuf.load(BWD && !a.Ua ? (const T*)a.dO + rowq * DV : vp + rowq * DV, (int64_t)H * DV, len);
  if (w == 0) {
    // gamma as hi + lo (two-sum scan); e^{gamma_L - gamma} from the exact
    // difference (e^gamma needs none: gamma's own rounding is relative to
    // gamma, and e^gamma is negligible wherever gamma is large)
    float glo;
    const float ghi = wave_incl_scan_2f(gv, glo);
    const float gLh = __shfl(ghi, 63, 64), gLl = __shfl(glo, 63, 64);
    const float eg = exp2_hw(ghi * LOG2E), eE = exp2_hw(((gLh - ghi) + (gLl - glo)) * LOG2E);
    sg[l] = ghi;
    sgl[l] = glo;
    sb[l] = bv;
    seg[l] = eg;
    sE[l] = eE;
    a.gam[ch * GSTRIDE + l] = ghi;
    a.gam[ch * GSTRIDE + 64 + l] = eg;
    a.gam[ch * GSTRIDE + 128 + l] = eE;
    a.gaml[ch * 64 + l] = glo;
  }
  kbuf.store(sK, LDK);
  GDR_SYNC();

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
        sA[r * LDF + s] = (s < r) ? sb[r] * acc[nt][i] * gate_factor<sizeof(T) == 4>(sg, sgl, r, s) : 0.f;
      }
  }
  GDR_SYNC();

  // T = (I + A)^-1 in place of A (A is zero on and above the diagonal, so
  // the strictly-upper blocks of T already are).  Diagonal 16 x 16 blocks by
  // forward substitution (wave 0: lane = (block, column); a wave's LDS
  // accesses are ordered, so every read of a block precedes its overwrite)
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
  GDR_SYNC();
  // off-diagonal block rows (fp32 MFMA, k = 4 per instruction): block row bi
  // reads A's blocks (bi, kb < bi), still intact, and T's rows above it;
  // T_{bi,j} replaces A_{bi,j} after the barrier that ends all reads of row bi
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
    GDR_SYNC();
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
    GDR_SYNC();
  }
  if constexpr (BWD) {
    // T in fp32, row-major, for the gradient kernel
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * (tid + 256 * q);
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sTm + (e >> 6) * LDF + (e & 63)), reinterpret_cast<f32x4*>(a.Tm + ch * 4096 + e));
    }
  }

  // W^T = K^T (T diag(beta e^gamma))^T (DK x 64): wave w owns dk rows
  // [w DK/4, (w+1) DK/4); T diag(beta e^gamma) is a split operand read from
  // the fp32 T.  Staged row-major in LDS (over A, which is dead), then
  // written out in fragment order.
  {
    constexpr int MT = DK / 64;
    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = zero4();
    auto d1 = [&](int s) { return sb[s] * seg[s]; };
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      frag af[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) af[mt] = frag_colk_lds(sK, LDK, w * (DK / 4) + 16 * mt, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        frag bh, bl;
        frag_rowk_f32<T>(sTm, LDF, 16 * nt, ks, d1, bh, bl);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][nt] = Mma<T>::mma(af[mt], bh, acc[mt][nt]);
          if constexpr (SPLIT) acc[mt][nt] = Mma<T>::mma(af[mt], bl, acc[mt][nt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) store_acc_t(sW, LDK, w * (DK / 4) + 16 * mt, 16 * nt, acc[mt][nt]);
  }
  GDR_SYNC();
  if (a.Wf) copy_afrag<T, 64, DK, false>((T*)a.Wf + ch * 64 * DK, sW, LDK);
  if constexpr (BWD) {
    copy_afrag<T, DK, 64, true>((T*)a.WTf + ch * DK * 64, sW, LDK);
    copy_afrag<T, 64, DK, false>((T*)a.Kf + ch * 64 * DK, sK, LDK);
  }
  if (a.KtTf) copy_afrag<T, DK, 64, true>((T*)a.KtTf + ch * DK * 64, sK, LDK);

  // U = T diag(beta) V per DV block (rows 16w, fp32, accumulator order);
  // T diag(beta) is a split operand read from the fp32 T.  The backward
  // needs U only to recompute the snapshots.
  if (!BWD || a.Ua) {
    auto d2 = [&](int s) { return sb[s]; };
    for (int dv0 = 0; dv0 < DV; dv0 += DVB) {
      GDR_SYNC();
      vbuf.store(sVu, LDV);
      if (dv0 + DVB < DV) vbuf.load(vp + rowq * DV + dv0 + DVB, (int64_t)H * DV, len);
      else if constexpr (BWD) vbuf.load((const T*)a.dO + rowq * DV, (int64_t)H * DV, len);   // first dO block
      GDR_SYNC();
      f32x4 acc[DVB / 16];
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt) acc[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 64; ks += KW) {
        frag ah, al;
        frag_rowk_f32<T>(sTm, LDF, 16 * w, ks, d2, ah, al);
#pragma unroll
        for (int nt = 0; nt < DVB / 16; ++nt) {
          const frag bv = frag_colk_lds(sVu, LDV, 16 * nt, ks);
          acc[nt] = Mma<T>::mma(ah, bv, acc[nt]);
          if constexpr (SPLIT) acc[nt] = Mma<T>::mma(al, bv, acc[nt]);
        }
      }
      float* Ub = a.Ua + ch * 64 * DV;
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt) store_acc4_nt(Ub + acc_off(w, dv0 / 16 + nt, DV), acc[nt]);
    }
  }

  GDR_SYNC();  // W staging, T and V are dead from here
  qbuf.store(sQ, LDK);
  GDR_SYNC();
  // forward: P = Q K^T * Gam (rows r = 16w); backward: P^T (rows s = 16w);
  // diagonal included, staged fp32 in its own orientation
  {
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
    const T* sA1 = BWD ? sK : sQ;
    const T* sB1 = BWD ? sQ : sK;
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const auto af = frag_rowk(sA1, LDK, 16 * w, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = Mma<T>::mma(af, frag_rowk(sB1, LDK, 16 * nt, ks), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 16 * w + acc_row0() + i, y = 16 * nt + acc_col();
        const int r = BWD ? y : x, s = BWD ? x : y;
        acc[nt][i] = (s <= r) ? acc[nt][i] * gate_factor<sizeof(T) == 4>(sg, sgl, r, s) : 0.f;
      }
      store_acc(sPT, LDF, 16 * w, 16 * nt, acc[nt]);
    }
  }
  GDR_SYNC();
  if constexpr (!BWD) {
    copy_afrag_split<T, 64, 64>((T*)a.Pf + ch * 4096, SPLIT ? (T*)a.Pfl + ch * 4096 : nullptr, sPT, LDF);
    copy_afrag<T, 64, DK, false>((T*)a.Qf + ch * 64 * DK, sQ, LDK);
  } else {
    // per DV block of dO: scale P^T dO (rows s = 16w) and scale Qg^T dO
    // (rows dk: wave w owns [w DK/4, (w+1) DK/4)), fp32, accumulator order;
    // P^T and Qg^T are split operands
    const float sc = a.scale;
    const T* dop = (const T*)a.dO;
    auto ps = [&](int) { return sc; };
    auto qs = [&](int r) { return sc * seg[r]; };
    constexpr int MT = DK / 64;
    for (int dv0 = 0; dv0 < DV; dv0 += DVB) {
      GDR_SYNC();
      vbuf.store(sVd, LDV);
      if (dv0 + DVB < DV) vbuf.load(dop + rowq * DV + dv0 + DVB, (int64_t)H * DV, len);
      GDR_SYNC();
      f32x4 accp[DVB / 16], accz[MT][DVB / 16];
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt) {
        accp[nt] = zero4();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) accz[mt][nt] = zero4();
      }
#pragma unroll
      for (int ks = 0; ks < 64; ks += KW) {
        frag ph, pl, qh[MT], ql[MT];
        frag_rowk_f32<T>(sPT, LDF, 16 * w, ks, ps, ph, pl);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) frag_colk_scaled<T>(sQ, LDK, w * (DK / 4) + 16 * mt, ks, qs, qh[mt], ql[mt]);
#pragma unroll
        for (int nt = 0; nt < DVB / 16; ++nt) {
          const frag bo = frag_colk_lds(sVd, LDV, 16 * nt, ks);
          accp[nt] = Mma<T>::mma(ph, bo, accp[nt]);
          if constexpr (SPLIT) accp[nt] = Mma<T>::mma(pl, bo, accp[nt]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            accz[mt][nt] = Mma<T>::mma(qh[mt], bo, accz[mt][nt]);
            if constexpr (SPLIT) accz[mt][nt] = Mma<T>::mma(ql[mt], bo, accz[mt][nt]);
          }
        }
      }
      float* Db = a.dDl + ch * 64 * DV;
      float* Zb = a.Z + ch * DK * DV;
#pragma unroll
      for (int nt = 0; nt < DVB / 16; ++nt) {
        store_acc4_nt(Db + acc_off(w, dv0 / 16 + nt, DV), accp[nt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) store_acc4_nt(Zb + acc_off(w * MT + mt, dv0 / 16 + nt, DV), accz[mt][nt]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_scan_fwd: per (unit, column tile).  Serial over the unit's chunks.  The
// state tile h (DK x DVT, fp32) is held in MFMA accumulators of waves 0..3
// (wave w owns dk rows [w DK/4, (w+1) DK/4)); h^T lives in LDS as a split
// operand (hi, lo) for W h and Q h.  Delta = U - W h and E Delta
// (E = e^{gamma_L - gamma}) go to LDS as split operands of P Delta and of
// the update h <- e^{gamma_L} h + K^T (E Delta).  All per-chunk operands
// that do not depend on h are loaded raw into a ring of SCAN_STAGES register
// sets, SCAN_STAGES - 1 chunks ahead; nothing touches a loaded value before
// its chunk is processed, so the loads stay in flight while earlier chunks
// run.  With the output fused and a ring of two or more stages, each role
// issues its prefetch while the other role issues none: the recurrence waves
// right after the first barrier (as the output waves form e^gamma Q h), the
// output waves right after the second (as the recurrence waves update h).
// The two roles' loads then do not queue behind each other in the compute
// unit's memory pipeline, whose issue rate bounds the chunk step (the loads
// for one chunk are ~68 KB per workgroup at 16-column tiles).  Without the
// output role (MODE 0, 1) the prefetch goes in three pieces spread over the
// step instead: W after the first barrier, K^T after the W h products, U and
// the gates after the second barrier.  With the output fused, each role
// runs a chunk loop of its own, chosen by a wave-uniform branch: the
// compiler's memory-wait analysis then sees only the role's own loads (with
// one loop for both, its paths ran the output waves' loads into the
// recurrence's registers and it waited for every load before the state
// update).
//   MODE 2: 8 waves.  Waves 0..3 run the recurrence and write the
//           snapshots; waves 4..7 compute o = scale (e^gamma (Q h) + P Delta)
//           beside them from double-buffered copies of h^T and Delta^T, so
//           the output is off the recurrence's critical path.  Both roles
//           meet at the same two barriers per chunk.
//   MODE 3: MODE 2 without the snapshots (forward calls that keep none);
//   MODE 1: writes the snapshots only (backward recompute);
//   MODE 0: CP segment summary -- scans the augmented state [I | 0] of width
//           DK + DV over one segment (the identity columns take U = 0, so
//           they evolve by the chunk transitions M_c alone) and writes the
//           final [prod M_c | state from zero] to the summary buffer.
// A unit is a (sequence, CP segment, head); segments other than the first
// start from the hand-off state, and only the last writes h_T.
#define SCAN_STAGES 3

template <typename T, typename HS, int DK, int DVT, int MODE>
__global__ __launch_bounds__(MODE >= 2 ? 512 : 256) void k_scan_fwd(const ScanFwdArgs a) {
  constexpr bool OUT = MODE >= 2;
  constexpr bool SNAP = MODE == 1 || MODE == 2;
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int P = pad_of<T>();
  constexpr int LDH = DK + P;
  constexpr int LDD = 64 + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int KS = DK / KW;
  constexpr int KS64 = 64 / KW;
  constexpr int MTH = DK / 64;
  constexpr int NT = DVT / 16;
  constexpr int NB = OUT ? 2 : 1;   // h^T / Delta^T buffers
  // fp32 fragments are 8x larger: shallower ring; 32-column snapshot tiles
  // take 2 stages and 64-column output tiles 2, so that two waves fit on
  // each SIMD
  constexpr int S = sizeof(T) == 2 ? ((OUT && DVT == 64) || (MODE == 1 && DVT == 32) ? 2 : SCAN_STAGES)
                                   : (OUT ? 1 : 2);
  // raw operand slots per ring stage, shared by both roles
  constexpr int NXR = KS + MTH * KS64;            // W, K^T
  constexpr int NXO = KS + (SPLIT ? 2 : 1) * KS64;  // Q, P (hi, lo)
  constexpr int NX = OUT ? cmax(NXR, NXO) : NXR;
  constexpr bool LATE = OUT && S >= 2;   // prefetch issued inside the chunk step
  constexpr bool SPREAD = !OUT && S >= 2;   // pieces spread over the step (no output role)
  typedef typename Mma<T>::frag frag;
  constexpr int LDO = DVT + P;
  __shared__ __align__(16) T sH[NB][DVT * LDH];                   // h^T (dv, dk), hi
  __shared__ __align__(16) T sHl[NB][SPLIT ? DVT * LDH : 1];      // lo
  __shared__ __align__(16) T sDE[DVT * LDD];                      // (E Delta)^T (dv, r), hi
  __shared__ __align__(16) T sDEl[SPLIT ? DVT * LDD : 1];
  __shared__ __align__(16) T sD[NB][OUT ? DVT * LDD : 1];         // Delta^T (dv, r), hi
  __shared__ __align__(16) T sDl[NB][OUT && SPLIT ? DVT * LDD : 1];
  __shared__ __align__(16) T sO[OUT ? 64 * LDO : 1];              // output staging

  const int H = a.geo.H, DV = a.DV, CP = a.geo.cp, N = a.geo.N;
  int p, jt;
  if (!unit_of(blockIdx.x, N * CP * H, a.ntiles, p, jt)) return;
  const int h = p % H, sg = (p / H) % CP, n = p / (H * CP);
  if (MODE == 0 && sg == CP - 1) return;   // the last segment hands nothing on
  const int col0 = jt * DVT;               // first column of the tile
  const bool mtile = MODE == 0 && col0 < DK;   // transition columns: start at I, no input
  const int dv0 = MODE == 0 ? (mtile ? 0 : col0 - DK) : col0;   // column of U (and o)
  int c0, nc, ts, tl;
  seg_range(a.geo, n, sg, c0, nc, ts, tl);
  const bool orole = OUT && wave_id() >= 4;   // output waves (wave-uniform)
  const int w = wave_id() & 3;                // row block of either role
  const int l = lane_id();
  const int dkw = w * (DK / 4);
  const int rw = 16 * w;
  const int64_t chb = (int64_t)h * a.geo.nchunks + c0;   // chunk-head index of chunk 0

  f32x4 acc_h[MTH][NT];
  const int64_t sb = (int64_t)(n * H + h) * DK * DV;
  const int64_t cpb = ((int64_t)sg * N * H + n * H + h) * DK;   // row 0 of this unit's CP tile
  if (!orole) {
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = dkw + 16 * mt + acc_row0() + i, dv = dv0 + 16 * nt + acc_col();
          float v = 0.f;
          if (MODE == 0) v = (mtile && dk == col0 + 16 * nt + acc_col()) ? 1.f : 0.f;
          else if (sg > 0) v = a.hstart[(cpb + dk) * DV + dv];
          else if (a.h0) v = (a.layout == 0) ? a.h0[sb + (int64_t)dk * DV + dv] : a.h0[sb + (int64_t)dv * DK + dk];
          acc_h[mt][nt][i] = v;
        }
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_acc_t2(sH[0], sHl[0], LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);
  }

  // one ring stage: recurrence waves hold W (x[0, KS)), K^T (x[KS, ..)),
  // U (v[0, NT)), E (v[NT]) and e^{gamma_L} (s); output waves hold Q
  // (x[0, KS)), P hi (x[KS, KS + KS64)), P lo (after it) and e^gamma (v[NT])
  struct Ops {
    frag x[NX];
    f32x4 v[NT + 1];
    float s;
  };
  // the recurrence's operands of load_ops in three pieces (W, K^T, U and the
  // gates), for the spread prefetch of MODE 0 and 1
  auto load_rpiece = [&](int c, Ops& o, int piece) {
    const int64_t ch = chb + c;
    const float* gb = a.gam + ch * GSTRIDE;
    if (piece == 0) {
      const T* Wb = (const T*)a.Wf + ch * 64 * DK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o.x[ks] = frag_af<T, DK>(Wb, w, ks);
    } else if (piece == 1) {
      const T* Kb = (const T*)a.KtTf + ch * DK * 64;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS64; ++ks) o.x[KS + mt * KS64 + ks] = frag_af<T, 64>(Kb, dkw / 16 + mt, ks);
    } else {
      const float* Ub = a.Ua + ch * 64 * DV;
      // U is read by this tile only: streaming loads
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o.v[nt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Ub + acc_off(w, dv0 / 16 + nt, DV)));
      o.v[NT] = *reinterpret_cast<const f32x4*>(gb + 128 + rw + acc_row0());
      o.s = gb[64 + 63];
    }
  };
  auto load_ops = [&](auto role, int c, Ops& o) {
    constexpr bool OR = decltype(role)::value;
    const int64_t ch = chb + c;
    const float* gb = a.gam + ch * GSTRIDE;
    if constexpr (!OR) {
      const T* Wb = (const T*)a.Wf + ch * 64 * DK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o.x[ks] = frag_af<T, DK>(Wb, w, ks);
      const T* Kb = (const T*)a.KtTf + ch * DK * 64;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS64; ++ks) o.x[KS + mt * KS64 + ks] = frag_af<T, 64>(Kb, dkw / 16 + mt, ks);
      const float* Ub = a.Ua + ch * 64 * DV;
      // U is read by this tile only: streaming loads
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o.v[nt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Ub + acc_off(w, dv0 / 16 + nt, DV)));
      o.v[NT] = *reinterpret_cast<const f32x4*>(gb + 128 + rw + acc_row0());
      o.s = gb[64 + 63];
    } else if constexpr (OUT) {
      const T* Qb = (const T*)a.Qf + ch * 64 * DK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o.x[ks] = frag_af<T, DK>(Qb, w, ks);
      const T* Pb = (const T*)a.Pf + ch * 4096;
#pragma unroll
      for (int ks = 0; ks < KS64; ++ks) o.x[KS + ks] = frag_af<T, 64>(Pb, w, ks);
      if constexpr (SPLIT) {
        const T* Pl = (const T*)a.Pfl + ch * 4096;
#pragma unroll
        for (int ks = 0; ks < KS64; ++ks) o.x[KS + KS64 + ks] = frag_af<T, 64>(Pl, w, ks);
      }
      o.v[NT] = *reinterpret_cast<const f32x4*>(gb + 64 + rw + acc_row0());
    }
  };

  // chunk c from stage o; with LATE and pf, the operands of chunk cn go to
  // stage on from inside the step
  auto process = [&](auto role, int c, Ops& o, int cn, Ops& on, bool pf) {
    constexpr bool OR = decltype(role)::value;
    const int64_t ch = chb + c;
    const int hb = OUT ? (c & 1) : 0;   // buffer holding h_c and Delta_c
    if constexpr (SNAP) {
      if constexpr (!OR) {
        HS* hsb = (HS*)a.hs + ch * DK * DV;
#pragma unroll
        for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) store_acc4_nt(hsb + acc_off(dkw / 16 + mt, dv0 / 16 + nt, DV), acc_h[mt][nt]);
      }
    }
    GDR_SYNC();  // h^T of this chunk is complete
    f32x4 acc_o[NT];
    if constexpr (!OR) {
      if (LATE && pf) {   // (the output waves': after the next barrier)
        __builtin_amdgcn_sched_barrier(0);
        load_ops(role, cn, on);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (SPREAD && pf) load_rpiece(cn, on, 0);
      // Delta = U - W h (rows 16w)
      f32x4 acc_d[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_d[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc_d[nt] = Mma<T>::mma(o.x[ks], frag_rowk(sH[hb], LDH, 16 * nt, ks * KW), acc_d[nt]);
          if constexpr (SPLIT) acc_d[nt] = Mma<T>::mma(o.x[ks], frag_rowk(sHl[hb], LDH, 16 * nt, ks * KW), acc_d[nt]);
        }
      if (SPREAD && pf) load_rpiece(cn, on, 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_d[nt][i] = (mtile ? 0.f : o.v[nt][i]) - acc_d[nt][i];
        store_acc_t2(sDE, sDEl, LDD, rw, 16 * nt, acc_d[nt] * o.v[NT]);
        if constexpr (OUT) store_acc_t2(sD[hb], sDl[hb], LDD, rw, 16 * nt, acc_d[nt]);
      }
    } else if constexpr (OUT) {
      // e^gamma (Q h) (rows 16w)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_o[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc_o[nt] = Mma<T>::mma(o.x[ks], frag_rowk(sH[hb], LDH, 16 * nt, ks * KW), acc_o[nt]);
          if constexpr (SPLIT) acc_o[nt] = Mma<T>::mma(o.x[ks], frag_rowk(sHl[hb], LDH, 16 * nt, ks * KW), acc_o[nt]);
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_o[nt] *= o.v[NT];
    }
    GDR_SYNC();  // Delta^T complete; all readers of the other h^T buffer are done
    if constexpr (OR) {
      if (LATE && pf) {
        __builtin_amdgcn_sched_barrier(0);
        load_ops(role, cn, on);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!OR) {
      if (SPREAD && pf) load_rpiece(cn, on, 2);
      // h <- e^{gamma_L} h + K^T (E Delta)
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc_h[mt][nt] *= o.s;
#pragma unroll
      for (int ks = 0; ks < KS64; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const frag be = frag_rowk(sDE, LDD, 16 * nt, ks * KW);
#pragma unroll
          for (int mt = 0; mt < MTH; ++mt) acc_h[mt][nt] = Mma<T>::mma(o.x[KS + mt * KS64 + ks], be, acc_h[mt][nt]);
          if constexpr (SPLIT) {
            const frag bel = frag_rowk(sDEl, LDD, 16 * nt, ks * KW);
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt) acc_h[mt][nt] = Mma<T>::mma(o.x[KS + mt * KS64 + ks], bel, acc_h[mt][nt]);
          }
        }
      const int hn = OUT ? (hb ^ 1) : 0;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) store_acc_t2(sH[hn], sHl[hn], LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);
    } else if constexpr (OUT) {
      // + P Delta, then write o: each output wave stages its 16 rows in LDS
      // and writes them back as 16-byte pieces (LDS accesses of one wave are
      // ordered: no barrier)
#pragma unroll
      for (int ks = 0; ks < KS64; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const frag bd = frag_rowk(sD[hb], LDD, 16 * nt, ks * KW);
          acc_o[nt] = Mma<T>::mma(o.x[KS + ks], bd, acc_o[nt]);
          if constexpr (SPLIT) {
            const frag bdl = frag_rowk(sDl[hb], LDD, 16 * nt, ks * KW);
            acc_o[nt] = Mma<T>::mma(o.x[KS + ks], bdl, acc_o[nt]);
            acc_o[nt] = Mma<T>::mma(o.x[KS + KS64 + ks], bd, acc_o[nt]);
          }
        }
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
  // each role runs a loop of its own (the same barriers, in the same order),
  // selected by a wave-uniform branch
  auto run = [&](auto role) {
    if (nc > 0) {
      Ops st[S];
#pragma unroll
      for (int s = 0; s < S - 1; ++s) load_ops(role, min(s, nc - 1), st[s]);
      int cb = 0;
      for (; cb + S <= nc; cb += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int cn = min(cb + s + S - 1, nc - 1);
          if (!LATE && !SPREAD) load_ops(role, cn, st[(s + S - 1) % S]);
          process(role, cb + s, st[s], cn, st[(s + S - 1) % S], true);
        }
      }
#pragma unroll
      for (int s = 0; s < S - 1; ++s)
        if (cb + s < nc) process(role, cb + s, st[s], 0, st[s], false);
    }
  };
  if (OUT && orole) run(std::integral_constant<bool, OUT>{});
  else run(std::false_type{});
  if (orole) return;
  if (MODE == 0) {
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = dkw + 16 * mt + acc_row0() + i;
          a.summ[(cpb + dk) * (DK + DV) + col0 + 16 * nt + acc_col()] = acc_h[mt][nt][i];
        }
  } else if (a.hT && sg == CP - 1) {
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
// k_cp_chain: per (sequence, head, 16-column tile).  Serial over the CP
// segments: X <- S X + Y with [S | Y] the segment summary (DK x (DK + 16)
// slice, fp32) and X the DK x 16 state slice in LDS; fp32 FMA throughout.
// Thread t owns column t % 16 and rows [(t / 16) DK/16, (t / 16 + 1) DK/16).
// The next segment's S is loaded into registers while the current hop
// computes, and stored to the other LDS buffer after it.
template <int DK>
__global__ __launch_bounds__(256) void k_cp_chain(const CpChainArgs a) {
  constexpr int LDM = DK + 4;   // keeps float4 rows 16-byte aligned
  constexpr int RPT = DK / 16;  // rows per thread
  constexpr int NPF = DK * DK / 4 / 256;   // float4 pieces of S per thread
  extern __shared__ __align__(16) char smem[];
  float* sM = (float*)smem;          // two buffers of S (r, m)
  float* sX = sM + 2 * DK * LDM;     // X (m, j)
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int H = a.geo.H, N = a.geo.N, CP = a.geo.cp, DV = a.DV;
  const int p = blockIdx.x, n = p / H, h = p - n * H;
  const int dv0 = blockIdx.y * 16;
  const int tid = threadIdx.x, j = tid & 15, r0 = (tid >> 4) * RPT;
  const int64_t sb = (int64_t)(n * H + h) * DK * DV;
  const int W = DK + DV;
  auto seg_of = [&](int it) { return a.bwd ? CP - 1 - it : it; };   // summary applied at hop it
  auto summ = [&](int s) { return a.summ + ((int64_t)s * N * H + n * H + h) * DK * W; };
  for (int e = tid; e < DK * 16; e += 256) {
    const int m = e >> 4, jj = e & 15;
    float v = 0.f;
    if (a.init) v = (a.layout == 0) ? a.init[sb + (int64_t)m * DV + dv0 + jj] : a.init[sb + (int64_t)(dv0 + jj) * DK + m];
    sX[m * 16 + jj] = v;
  }
  f4 pf[NPF];
  auto fetch = [&](int s) {
    const float* Sb = summ(s);
#pragma unroll
    for (int q = 0; q < NPF; ++q) {
      const int e = tid + 256 * q, r = e / (DK / 4), c = (e - r * (DK / 4)) * 4;
      pf[q] = *reinterpret_cast<const f4*>(Sb + (int64_t)r * W + c);
    }
  };
  auto stash = [&](float* dst) {
#pragma unroll
    for (int q = 0; q < NPF; ++q) {
      const int e = tid + 256 * q, r = e / (DK / 4), c = (e - r * (DK / 4)) * 4;
      *reinterpret_cast<f4*>(dst + r * LDM + c) = pf[q];
    }
  };
  fetch(seg_of(0));
  stash(sM);
  for (int it = 0; it < CP - 1; ++it) {
    const int s = seg_of(it);
    const int so = a.bwd ? s - 1 : s + 1;          // segment whose state is produced
    const float* M = sM + (it & 1) * DK * LDM;
    if (it + 1 < CP - 1) fetch(seg_of(it + 1));
    float acc[RPT];
    const float* Sb = summ(s);
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = Sb[(int64_t)(r0 + r) * W + DK + dv0 + j];
    GDR_SYNC();  // S in this buffer and X are complete
    for (int m = 0; m < DK; m += 4) {
      const float x0 = sX[m * 16 + j], x1 = sX[(m + 1) * 16 + j];
      const float x2 = sX[(m + 2) * 16 + j], x3 = sX[(m + 3) * 16 + j];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const f4 mv = *reinterpret_cast<const f4*>(M + (r0 + r) * LDM + m);
        acc[r] = fmaf(mv[0], x0, acc[r]);
        acc[r] = fmaf(mv[1], x1, acc[r]);
        acc[r] = fmaf(mv[2], x2, acc[r]);
        acc[r] = fmaf(mv[3], x3, acc[r]);
      }
    }
    GDR_SYNC();  // all reads of X and of this S buffer done
    if (it + 1 < CP - 1) stash(sM + ((it + 1) & 1) * DK * LDM);
    float* ob = a.out + ((int64_t)so * N * H + n * H + h) * DK * DV;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      sX[(r0 + r) * 16 + j] = acc[r];
      ob[(int64_t)(r0 + r) * DV + dv0 + j] = acc[r];
    }
  }
}

// ---------------------------------------------------------------------------
// host-side launchers

template <typename T, int DK, bool BWD>
static size_t wy_smem() {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P, LDF = 68, DVB = dvb_of<T>(), LDV = DVB + P;
  constexpr int R2 = cmax(64 * LDK * (int)sizeof(T), cmax(64 * LDV * (int)sizeof(T), 4 * 16 * 20 * 4));
  return 64 * LDK * sizeof(T) + 64 * LDF * 4 + R2 + 5 * 64 * 4;
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

// ---------------------------------------------------------------------------
// k_check_cu: one workgroup of 1024 threads checks the packed-batch contract
// of cu_seqlens (cu[0] = 0, every later entry in [previous entry, T_total])
// and writes to *result the smallest index of an entry that breaks it, or -1.
// The kernel writes its result unconditionally, so the buffer needs no
// clearing beforehand.
__global__ __launch_bounds__(1024) void k_check_cu(const int* cu, int N, int T_total, int* result) {
  __shared__ int s_min[1024];
  const int tid = threadIdx.x;
  int bad = INT_MAX;
  for (int i = tid; i <= N; i += 1024) {
    const int c = cu[i];
    const bool ok = i == 0 ? c == 0 : (c >= cu[i - 1] && c <= T_total);
    if (!ok) bad = min(bad, i);
  }
  s_min[tid] = bad;
  GDR_SYNC();
  for (int d = 512; d > 0; d >>= 1) {
    if (tid < d) s_min[tid] = min(s_min[tid], s_min[tid + d]);
    GDR_SYNC();
  }
  if (tid == 0) *result = s_min[0] == INT_MAX ? -1 : s_min[0];
}

hipError_t launch_check_cu(const int* cu, int N, int T_total, int* result, hipStream_t st) {
  hipLaunchKernelGGL(k_check_cu, dim3(1), dim3(1024), 0, st, cu, N, T_total, result);
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

template <typename T, typename HS, int DK, int MODE>
static hipError_t launch_scan_fwd_t(ScanFwdArgs a, int dvt, hipStream_t st) {
  const int units = a.geo.N * a.geo.cp * a.geo.H;
  a.ntiles = ((MODE == 0 ? DK : 0) + a.DV) / dvt;
  const int grid = 8 * ((units + 7) / 8) * a.ntiles;
  if (units == 0) return hipSuccess;
  const int nthr = MODE >= 2 ? 512 : 256;
  if (dvt == 16) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 16, MODE>), dim3(grid), dim3(nthr), 0, st, a);
  else if constexpr (sizeof(T) == 2) {
    if (dvt == 32) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 32, MODE>), dim3(grid), dim3(nthr), 0, st, a);
    else if constexpr (MODE >= 2) {   // 64-column tiles: output scans only
      if (dvt == 64) hipLaunchKernelGGL((k_scan_fwd<T, HS, DK, 64, MODE>), dim3(grid), dim3(nthr), 0, st, a);
      else return hipErrorInvalidValue;
    }
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, typename HS, int DK>
static hipError_t launch_scan_fwd_m(const ScanFwdArgs& a, int dvt, int mode, hipStream_t st) {
  if (mode == 0) return launch_scan_fwd_t<T, float, DK, 0>(a, dvt, st);   // no snapshots: HS unused
  if (mode == 1) return launch_scan_fwd_t<T, HS, DK, 1>(a, dvt, st);
  if (mode == 3) return launch_scan_fwd_t<T, float, DK, 3>(a, dvt, st);  // no snapshots: HS unused
  return launch_scan_fwd_t<T, HS, DK, 2>(a, dvt, st);
}

template <typename T, typename HS>
static hipError_t launch_scan_fwd_d(const ScanFwdArgs& a, int DK, int dvt, int mode, hipStream_t st) {
  if (DK == 64) return launch_scan_fwd_m<T, HS, 64>(a, dvt, mode, st);
  return launch_scan_fwd_m<T, HS, 128>(a, dvt, mode, st);
}

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool f32, int hs_dtype, int DK, int dvt, int mode, hipStream_t st) {
  if (f32) return launch_scan_fwd_d<float, float>(a, DK, dvt, mode, st);
  if (hs_dtype == GDR_F32) return launch_scan_fwd_d<bf16, float>(a, DK, dvt, mode, st);
  if (hs_dtype == GDR_F16) return launch_scan_fwd_d<bf16, f16>(a, DK, dvt, mode, st);
  return launch_scan_fwd_d<bf16, bf16>(a, DK, dvt, mode, st);
}

template <int DK>
static hipError_t launch_cp_chain_t(const CpChainArgs& a, hipStream_t st) {
  const size_t sm = (size_t)(2 * DK * (DK + 4) + DK * 16) * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)k_cp_chain<DK>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_cp_chain<DK>, dim3(a.geo.N * a.geo.H, a.DV / 16), dim3(256), sm, st, a);
  return hipGetLastError();
}

hipError_t launch_cp_chain(const CpChainArgs& a, hipStream_t st) {
  if (a.geo.N * a.geo.H == 0 || a.geo.cp <= 1) return hipSuccess;
  return a.DK == 64 ? launch_cp_chain_t<64>(a, st) : launch_cp_chain_t<128>(a, st);
}

#ifdef GDR_DEBUG_DELAY
// the race-test build: this file's copy of the barrier-delay settings
hipError_t debug_set_delay_fwd(const DelayCfg& c) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_delay), &c, sizeof(c));
}
#endif

}  // namespace gdr
