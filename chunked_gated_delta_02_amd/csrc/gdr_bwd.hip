// gdr_bwd.hip -- backward kernels of the chunked gated delta rule on gfx950
// (the fused backward that FlashQLA PR #34, "SM120/121 : Add support for
// fused backward kernel", section "Summary", calls fused_gdr_bwd).
//
// Reverse-mode differentiation of the chunk-wise forward (see gdr_fwd.hip),
// per chunk with state h at its start, dh = gradient of the state at its end
// and dO, all in KV form:
//   dDelta  = scale P^T dO + Kt dh                    (P = Q K^T * Gam)
//   dh_prev = scale Qg^T dO + e^{gamma_L} dh - W^T dDelta    (Qg = e^gamma Q)
//   dq  = e^gamma (scale dO h^T) + (dP * Gam) K,      dP = scale dO Delta^T
//   dk  = E (Delta dh^T) + (dP * Gam)^T Q + beta e^gamma (T^T dW)
//         + G K + G^T K,        E = e^{gamma_L - gamma}, dW = -dDelta h^T,
//                               G = dA * beta Gam (strictly lower)
//   dv  = beta (T^T dDelta)
//   dA  = strictly_lower(-T^T dT T^T),  dT = dDelta (beta V)^T + dW (beta e^gamma K)^T
//   dbeta = rowsum(V * T^T dDelta) + e^gamma rowsum(K * T^T dW) + rowsum(dA * K K^T * Gam)
//   dgamma collects e^gamma rowsum(Q * scale dO h^T), rowsum - colsum of
//   dP * P and dA * A, -rowsum(K * E Delta dh^T) (plus its sum into gamma_L),
//   beta e^gamma rowsum(K * T^T dW) and e^{gamma_L} <dh, h> into gamma_L;
//   dg is the chunk-local reverse cumulative sum of dgamma.
// Sums across tiles run in a fixed order (no floating-point atomics), so
// results are bitwise reproducible -- the determinism requirement argued in
// Dao-AILab/quack PR #101 ("Rmsnorm backward fusing sum", review thread).
//
// Kernels:
//   k_scan_bwd  serial over chunks (last to first) per (sequence, head, DV
//               tile): dh lives in fp32 MFMA accumulators; writes the per-chunk
//               dh snapshot, dDelta and dh0.
//   k_grad      chunk-parallel: every intra-chunk gradient GEMM, the WY/UT
//               backward and the dbeta / dg reductions, in one kernel.
#include "gdr_kernels.h"

namespace gdr {

// ---------------------------------------------------------------------------
// k_scan_bwd: per (unit, column tile), chunks last to first.  dh (the
// gradient of the state at the chunk's end, DK x DVT fp32) lives in MFMA
// accumulators; dh^T in LDS is a split operand (hi, lo) of K dh.  Per chunk
//   dDelta = E (K dh) + scale P^T dO          (E scales rows; K exact)
//   dh    <- e^{gamma_L} dh + scale Qg^T dO - W^T dDelta
// where the two dh-independent terms come precomputed in fp32 and
// -dDelta^T goes to LDS as a split operand.  The per-chunk operands (K,
// W^T, the two fp32 terms, the gate factors) are loaded raw into a ring of
// SCAN_STAGES register sets, SCAN_STAGES - 1 chunks ahead; each chunk issues
// the next loads in pieces spread over its step (K after the first barrier,
// W^T after the K dh products, the fp32 terms and gates between the MFMA
// steps of the dh update), so that the compute unit's memory pipeline, whose
// issue rate bounds the step, drains between them.  Writes the dh
// snapshot and dDelta (io dtype; the gradient kernel rounds its MFMA
// operands to it anyway), both in accumulator order, and dh0.  These two
// are written with ordinary stores: the gradient kernel reads them right
// after this kernel and finds them in the Infinity Cache (measured faster
// than streaming stores, which leave the scan itself unchanged).
//   MODE 1: the reverse scan proper.
//   MODE 0: CP segment summary -- scans the augmented gradient [I | 0] of
//           width DK + DV backwards over one segment (the identity columns
//           take no dO terms, so they evolve by the transposed transitions
//           alone) and writes [prod M_c^T | gradient from zero] at the
//           segment start.
// A unit is a (sequence, CP segment, head); segments other than the last
// start from the hand-off gradient, and only the first writes dh0.
#define SCAN_STAGES 3

template <typename T, int DK, int DVT, int MODE>
__global__ __launch_bounds__(256) void k_scan_bwd(const ScanBwdArgs a) {
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int P = pad_of<T>();
  constexpr int LDH = DK + P;
  constexpr int LDD = 64 + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int KS = DK / KW;
  constexpr int KS64 = 64 / KW;
  constexpr int MTH = DK / 64;
  constexpr int NT = DVT / 16;
  // fp32 fragments are 8x larger; 32-column tiles take a 2-stage ring so
  // that two waves fit on each SIMD
  constexpr int S = sizeof(T) == 2 ? (DVT == 32 ? 2 : SCAN_STAGES) : 2;
  typedef typename Mma<T>::frag frag;
  __shared__ __align__(16) T sDH[DVT * LDH];               // dh^T (dv, dk), hi
  __shared__ __align__(16) T sDHl[SPLIT ? DVT * LDH : 1];  // lo
  __shared__ __align__(16) T sDD[DVT * LDD];               // -dDelta^T (dv, r), hi
  __shared__ __align__(16) T sDDl[SPLIT ? DVT * LDD : 1];  // lo

  const int H = a.geo.H, DV = a.DV, CP = a.geo.cp, N = a.geo.N;
  int p, jt;
  if (!unit_of(blockIdx.x, N * CP * H, a.ntiles, p, jt)) return;
  const int h = p % H, sg = (p / H) % CP, n = p / (H * CP);
  if (MODE == 0 && sg == 0) return;        // the first segment hands nothing back
  const int col0 = jt * DVT;
  const bool mtile = MODE == 0 && col0 < DK;   // transition columns: start at I, no dO
  const int dv0 = MODE == 0 ? (mtile ? 0 : col0 - DK) : col0;   // column of the dO terms
  int c0, nc, ts, tl;
  seg_range(a.geo, n, sg, c0, nc, ts, tl);
  const int w = wave_id();
  const int dkw = w * (DK / 4);
  const int rw = 16 * w;
  const int64_t chb = (int64_t)h * a.geo.nchunks + c0;

  f32x4 acc_h[MTH][NT];
  const int64_t sb = (int64_t)(n * H + h) * DK * DV;
  const int64_t cpb = ((int64_t)sg * N * H + n * H + h) * DK;
#pragma unroll
  for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = dkw + 16 * mt + acc_row0() + i, dv = dv0 + 16 * nt + acc_col();
        float v = 0.f;
        if (MODE == 0) v = (mtile && dk == col0 + 16 * nt + acc_col()) ? 1.f : 0.f;
        else if (sg < CP - 1) v = a.dhend[(cpb + dk) * DV + dv];
        else if (a.dhT) v = (a.layout == 0) ? a.dhT[sb + (int64_t)dk * DV + dv] : a.dhT[sb + (int64_t)dv * DK + dk];
        acc_h[mt][nt][i] = v;
      }
#pragma unroll
  for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) store_acc_t2(sDH, sDHl, LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);

  struct Ops {
    frag kf[KS];            // K rows 16w (rows >= len are zero)
    frag wf[MTH][KS64];     // W^T rows dkw..
    f32x4 dl[NT];           // scale P^T dO (fp32, accumulator order, raw)
    f32x4 z[MTH][NT];       // scale Qg^T dO (fp32, accumulator order, raw)
    f32x4 ee;               // e^{gamma_L - gamma} of the lane's 4 rows
    float eL;               // e^{gamma_L}
  };
  // the operands of chunk c in four pieces: K, W^T, the fp32 terms, gates
  auto load_piece = [&](int c, Ops& o, int piece) {
    const int64_t ch = chb + c;
    if (piece == 0) {
      const T* Kb = (const T*)a.Kf + ch * 64 * DK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o.kf[ks] = frag_af<T, DK>(Kb, w, ks);
    } else if (piece == 1) {
      const T* Wb = (const T*)a.WTf + ch * DK * 64;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS64; ++ks) o.wf[mt][ks] = frag_af<T, 64>(Wb, dkw / 16 + mt, ks);
    } else if (piece == 2) {
      // the two fp32 terms are read by this tile only: streaming loads
      const float* Db = a.dDl + ch * 64 * DV;
      const float* Zb = a.Z + ch * DK * DV;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        o.dl[nt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Db + acc_off(w, dv0 / 16 + nt, DV)));
#pragma unroll
        for (int mt = 0; mt < MTH; ++mt)
          o.z[mt][nt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Zb + acc_off(dkw / 16 + mt, dv0 / 16 + nt, DV)));
      }
    } else {
      const float* gb = a.gam + ch * GSTRIDE;
      o.ee = *reinterpret_cast<const f32x4*>(gb + 128 + rw + acc_row0());
      o.eL = gb[64 + 63];
    }
  };

  // L2 warming (16-bit operands).  The column tiles of a unit run in step
  // and share its K and W^T fragments through their XCD's L2, but they
  // request each chunk at the same moment, so every one of them waits for
  // the HBM fill.  Each wave also touches one 1 KB fragment of its tile's
  // share of the chunk WARM steps ahead (fragment jt + ntiles * wave of the
  // 2 NKF K and W^T fragments; one dword per lane at a 16-byte stride reaches
  // every line of it), so that the ring's loads of that chunk hit L2.  The
  // value is consumed by an empty asm one step later, where the compiler's
  // wait covers it.  At 8 or more tiles every shared fragment is warmed.
  // 16-column tiles only: at 32 columns (a 2-stage ring, two waves per
  // SIMD) the extra loads cost more than they save (B = 4, T = 8192, H = 32,
  // DV = 256: 993 -> 1061 us), at 16 they save (B = 2, T = 4096, H = 16:
  // 106.6 -> 102.1 us).
  constexpr int WARM = 6;
  constexpr int NKF = 64 * DK / 512;
  float wcarry = 0.f;
  auto warm = [&](int c) {
    if constexpr (sizeof(T) == 2 && DVT == 16) {
      asm volatile("" ::"v"(wcarry));
      const int64_t ch = chb + max(c - WARM, 0);
      const int q = (jt + a.ntiles * w) % (2 * NKF);
      const T* base = q < NKF ? (const T*)a.Kf + ch * 64 * DK : (const T*)a.WTf + ch * DK * 64;
      const int f = q < NKF ? q : q - NKF;
      wcarry = *reinterpret_cast<const float*>(base + ((int64_t)f * 64 + lane_id()) * 8);
    }
  };

  // chunk c from stage o; with pf, the operands of chunk cn go to stage on
  auto process = [&](int c, Ops& o, int cn, Ops& on, bool pf) {
    const int64_t ch = chb + c;
    if constexpr (MODE != 0) {
      T* db = (T*)a.dhs + ch * DK * DV;
#pragma unroll
      for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) store_acc4(db + acc_off(dkw / 16 + mt, dv0 / 16 + nt, DV), acc_h[mt][nt]);
    }
    GDR_SYNC();  // dh^T complete; last chunk's readers of dDelta^T are done
    if (pf) {
      __builtin_amdgcn_sched_barrier(0);
      load_piece(cn, on, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dDelta = E (K dh) + scale P^T dO, rows 16w
    f32x4 acc_d[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc_d[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc_d[nt] = Mma<T>::mma(o.kf[ks], frag_rowk(sDH, LDH, 16 * nt, ks * KW), acc_d[nt]);
        if constexpr (SPLIT) acc_d[nt] = Mma<T>::mma(o.kf[ks], frag_rowk(sDHl, LDH, 16 * nt, ks * KW), acc_d[nt]);
      }
    if (pf) {
      __builtin_amdgcn_sched_barrier(0);
      load_piece(cn, on, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc_d[nt] = acc_d[nt] * o.ee + (mtile ? zero4() : o.dl[nt]);
      if constexpr (MODE != 0) store_acc4((T*)a.dD + ch * 64 * DV + acc_off(w, dv0 / 16 + nt, DV), acc_d[nt]);
      store_acc_t2(sDD, sDDl, LDD, rw, 16 * nt, -acc_d[nt]);
    }
    GDR_SYNC();  // -dDelta^T complete; all readers of dh^T are done
    // dh <- e^{gamma_L} dh + scale Qg^T dO - W^T dDelta
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc_h[mt][nt] = acc_h[mt][nt] * o.eL + (mtile ? zero4() : o.z[mt][nt]);
#pragma unroll
    for (int ks = 0; ks < KS64; ++ks) {
      // the rest of the prefetch goes between these MFMA steps, where its
      // issue overlaps the MFMA chain instead of delaying the next barrier
      if (pf) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) warm(c);
#pragma unroll
        for (int pc = 2; pc < 4; ++pc)
          if ((pc - 2) * KS64 / 2 == ks) load_piece(cn, on, pc);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const frag bd = frag_rowk(sDD, LDD, 16 * nt, ks * KW);
#pragma unroll
        for (int mt = 0; mt < MTH; ++mt) acc_h[mt][nt] = Mma<T>::mma(o.wf[mt][ks], bd, acc_h[mt][nt]);
        if constexpr (SPLIT) {
          const frag bdl = frag_rowk(sDDl, LDD, 16 * nt, ks * KW);
#pragma unroll
          for (int mt = 0; mt < MTH; ++mt) acc_h[mt][nt] = Mma<T>::mma(o.wf[mt][ks], bdl, acc_h[mt][nt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) store_acc_t2(sDH, sDHl, LDH, dkw + 16 * mt, 16 * nt, acc_h[mt][nt]);
  };

  // Chunks are processed last to first: step j handles chunk nc - 1 - j and
  // lives in register stage j % S.  As in the forward scan, the main loop
  // runs S steps per trip with unconditional prefetches (index clamped to
  // the first chunk) so the prefetched loads stay in flight, and a static
  // tail runs the last nc % S steps.
  if (nc > 0) {
    Ops st[S];
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) load_piece(nc - 1 - min(s, nc - 1), st[s], pc);
    int jb = 0;
    for (; jb + S <= nc; jb += S) {
#pragma unroll
      for (int s = 0; s < S; ++s)
        process(nc - 1 - (jb + s), st[s], nc - 1 - min(jb + s + S - 1, nc - 1), st[(s + S - 1) % S], true);
    }
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (jb + s < nc) process(nc - 1 - (jb + s), st[s], 0, st[s], false);
  }
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
  } else if (a.dh0 && sg == 0) {
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = dkw + 16 * mt + acc_row0() + i, dv = dv0 + 16 * nt + acc_col();
          if (a.layout == 0) a.dh0[sb + (int64_t)dk * DV + dv] = acc_h[mt][nt][i];
          else a.dh0[sb + (int64_t)dv * DK + dk] = acc_h[mt][nt][i];
        }
  }
}

// value columns per phase-1 step of k_grad (keeps its LDS at two workgroups
// per compute unit)
#define GRAD_DVB 32

// ---------------------------------------------------------------------------
// k_grad: per (chunk, head).  Phase 1 loops over DV in blocks of DVB and
// accumulates the DV-contracted products (dQg, dKt, dW, dP, dT_V) in
// registers while emitting dv; phase 2 finishes dq, dk, dbeta and dg.  Any
// of dq, dk, dv, dbeta, dg may be null: its stores are then dropped (empty
// buffer range) or skipped; the computation is the same.  Wave w owns output
// rows 16w..16w+15 of every 64-row product, so all row sums stay inside one
// wavefront; column sums go through per-wave LDS partials reduced in a fixed
// order.  dVb (which becomes dv) is accumulated transposed (operands
// swapped, see tr_row): each lane holds four consecutive columns of one row,
// so a dv tile leaves in one 8-byte store per lane instead of four 2-byte
// ones and beta is one factor per lane.  (dq and dk taken the same way
// measured slower: the longer-lived row-major operands they need spill.)
template <typename T, typename HS, int DK>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k_grad(const GradArgs a) {
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P;
  constexpr int L64 = 64 + P;
  constexpr int DVB = GRAD_DVB;
  constexpr int LDV = DVB + P;
  constexpr int KW = Mma<T>::KW;
  constexpr int NTK = DK / 16;
  constexpr int NTB = DVB / 16;
  typedef typename Mma<T>::frag frag;
  constexpr int PH1 = (2 * DVB * LDK + 3 * DVB * L64 + 64 * LDV + DK * L64) * (int)sizeof(T);
  constexpr int PH2 = (2 * 64 * LDK + DK * L64 + 64 * L64) * (int)sizeof(T);
  extern __shared__ __align__(16) char smem[];
  T* sT = (T*)smem;                       // T (r, s), operand copy
  float* sg = (float*)(sT + 64 * L64);    // gamma (hi)
  float* sb = sg + 64;                    // beta
  float* seg = sb + 64;                   // e^gamma
  float* sE = seg + 64;                   // e^{gamma_L - gamma}
  float* sgl = sE + 64;                   // gamma (lo)
  float* sRed = sgl + 64;                 // [2][4][64] column-sum partials
  float* sMisc = sRed + 2 * 4 * 64;       // [8]: per-wave gamma_L partials
  char* uni = (char*)(sMisc + 8);
  // phase 1
  T* sHvk = (T*)uni;                      // h rows (dv, dk)
  T* sDHvk = sHvk + DVB * LDK;            // dh rows (dv, dk)
  T* sDeltaT = sDHvk + DVB * LDK;         // Delta^T (dv, r), hi
  T* sDeltaTl = sDeltaT + DVB * L64;      // lo
  T* sDDt = sDeltaTl + DVB * L64;         // dDelta^T (dv, r)
  T* sV = sDDt + DVB * L64;               // V (r, dv)
  T* sWT = sV + 64 * LDV;                 // W^T (dk, r)
  // phase 2 (aliases phase 1)
  T* sQ = (T*)uni;                        // Q (r, dk); later dT^T (s, r)
  T* sK = sQ + 64 * LDK;                  // K (r, dk)
  T* sdWT = sK + 64 * LDK;                // dW^T (dk, r); later G^T (c, a)
  T* sdQKT = sdWT + DK * L64;             // (dP * Gam)^T (s, r); later Y^T (b, a)
  static_assert(PH1 > 0 && PH2 > 0, "");

  const int ci = blockIdx.x, h = blockIdx.y;
  int n, t0, len;
  if (!chunk_lookup(a.geo, ci, n, t0, len)) return;
  const int H = a.geo.H, DV = a.DV;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t ch = (int64_t)h * a.geo.nchunks + ci;
  const T* qp = (const T*)a.q;
  const T* kp = (const T*)a.k;
  const T* vp = (const T*)a.v;
  const T* dop = (const T*)a.dO;
  const float scale = a.scale;

  if (tid < 64) {
    sg[tid] = a.gam[ch * GSTRIDE + tid];
    sgl[tid] = a.gaml[ch * 64 + tid];
    sb[tid] = (tid < len) ? a.beta[(int64_t)(t0 + tid) * H + h] : 0.f;
    seg[tid] = a.gam[ch * GSTRIDE + 64 + tid];
    sE[tid] = a.gam[ch * GSTRIDE + 128 + tid];
  }
  const float* Tg = a.Tm + ch * 4096;   // T, fp32 row-major
  {
    // T -> operand copy in the io dtype in LDS; W^T from fragment order into
    // (dk, r) rows in LDS; all loads issued first
    constexpr int KPL = Mma<T>::KPL;
    constexpr int WPT = (DK / 16) * (64 / KW) * 64 / 256;   // W^T fragment lanes per thread
    f32x4 tv[4];
    frag wv[WPT];
    const T* Wb = (const T*)a.WTf + ch * DK * 64;
#pragma unroll
    for (int q = 0; q < 4; ++q) tv[q] = *reinterpret_cast<const f32x4*>(Tg + 4 * (tid + 256 * q));
#pragma unroll
    for (int q = 0; q < WPT; ++q) wv[q] = *reinterpret_cast<const frag*>(Wb + (int64_t)(tid + 256 * q) * KPL);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * (tid + 256 * q);
      store_acc4(sT + (e >> 6) * L64 + (e & 63), tv[q]);
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int e = tid + 256 * q, f = e >> 6, ll = e & 63;
      const int m = f / (64 / KW), ks = f - m * (64 / KW);
      *reinterpret_cast<frag*>(sWT + (16 * m + (ll & 15)) * L64 + ks * KW + KPL * (ll >> 4)) = wv[q];
    }
  }
  const int rw = 16 * w;            // first output row of this wave
  const int r0 = rw + acc_row0();   // lane's rows r0..r0+3 (accumulator tiles)
  const int rs = rw + tr_row();     // lane's row in transposed tiles
  const int tc0 = tr_col0();        // and its first column there

  // per-lane row partials for the lane's 4 rows
  float rg[4] = {0.f, 0.f, 0.f, 0.f};   // dgamma row terms
  float rb[4] = {0.f, 0.f, 0.f, 0.f};   // dbeta row terms
  float rbS = 0.f;                      // dbeta terms of row rs (transposed tiles)
  float gLh = 0.f;                      // <dh, h> partial (times e^{gamma_L} later)
  float gLy = 0.f;                      // sum of E rowsum(K * Delta dh^T) partial

  // T diag(beta) (rows 16w) as a split operand of U = T diag(beta) V, read
  // from the fp32 T once the gates are in LDS
  GDR_SYNC();
  frag tbh[64 / KW], tbl[64 / KW];
#pragma unroll
  for (int ks = 0; ks < 64 / KW; ++ks) frag_rowk_f32<T>(Tg, 64, rw, ks * KW, [&](int s2) { return sb[s2]; }, tbh[ks], tbl[ks]);
  f32x4 aQ[NTK], aKt[NTK], aW[NTK], aP[4], aTV[4];
#pragma unroll
  for (int nt = 0; nt < NTK; ++nt) aQ[nt] = aKt[nt] = aW[nt] = zero4();
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) aP[nt] = aTV[nt] = zero4();

  const int64_t rowq = (int64_t)t0 * H + h;   // token-row index of chunk row 0
  for (int dvb = 0; dvb < DV; dvb += DVB) {
    frag dof[DVB / KW];     // dO fragments (rows 16w, k = dv)
    GDR_SYNC();
    // h and dh (accumulator order <DK, DV>) and dDelta (accumulator order
    // <64, DV>) of this DV block, transposed into (dv, .) rows in LDS;
    // <dh, h> (for e^{gamma_L} <dh, h>) uses h in its stored precision
    {
      // all global loads of this block are issued before the first LDS store
      const HS* hb = (const HS*)a.hs + ch * DK * DV;
      const T* db = (const T*)a.dhs + ch * DK * DV;
      const T* ddb = (const T*)a.dD + ch * 64 * DV;
      constexpr int IH = (DK / 16) * NTB * 64 / 256, ID = 4 * NTB * 64 / 256;
      typedef T t4 __attribute__((ext_vector_type(4)));
      f32x4 hv[IH];
      t4 gv[IH], dv4[ID];   // dh snapshot and dDelta, io dtype
      {
        const __amdgpu_buffer_rsrc_t rdo = buf_rsrc(dop + rowq * DV + dvb, len * H * DV * (int)sizeof(T));
#pragma unroll
        for (int ks = 0; ks < DVB / KW; ++ks)
          dof[ks] = frag_rowk_buf<T>(rdo, H * DV, rw, ks * KW);
      }
#pragma unroll
      for (int q = 0; q < IH; ++q) {
        const int e = tid + 256 * q, ll = e & 63, tt = e >> 6;
        const int m = tt / NTB, nn = tt - m * NTB;
        const int64_t off = acc_off_l(m, dvb / 16 + nn, DV, ll);
        // the snapshots are read by this workgroup only: streaming loads
        if constexpr (sizeof(HS) == 4) hv[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hb + off));
        else hv[q] = load4f(hb + off);
        gv[q] = __builtin_nontemporal_load(reinterpret_cast<const t4*>(db + off));
      }
#pragma unroll
      for (int q = 0; q < ID; ++q) {
        const int e = tid + 256 * q, ll = e & 63, tt = e >> 6;
        const int m = tt / NTB, nn = tt - m * NTB;
        dv4[q] = __builtin_nontemporal_load(reinterpret_cast<const t4*>(ddb + acc_off_l(m, dvb / 16 + nn, DV, ll)));
      }
#pragma unroll
      for (int q = 0; q < IH; ++q) {
        const int e = tid + 256 * q, ll = e & 63, tt = e >> 6;
        const int m = tt / NTB, nn = tt - m * NTB;
        const int dk = 16 * m + 4 * (ll >> 4), dvl = 16 * nn + (ll & 15);
        const f32x4 g4 = {to_f32(gv[q][0]), to_f32(gv[q][1]), to_f32(gv[q][2]), to_f32(gv[q][3])};
        gLh += hv[q][0] * g4[0] + hv[q][1] * g4[1] + hv[q][2] * g4[2] + hv[q][3] * g4[3];
        store_acc4(sHvk + dvl * LDK + dk, hv[q]);
        *reinterpret_cast<t4*>(sDHvk + dvl * LDK + dk) = gv[q];
      }
#pragma unroll
      for (int q = 0; q < ID; ++q) {
        const int e = tid + 256 * q, ll = e & 63, tt = e >> 6;
        const int m = tt / NTB, nn = tt - m * NTB;
        const int r = 16 * m + 4 * (ll >> 4), dvl = 16 * nn + (ll & 15);
        *reinterpret_cast<t4*>(sDDt + dvl * L64 + r) = dv4[q];
      }
    }
    load_rows<T, DVB>(sV, LDV, vp + rowq * DV + dvb, (int64_t)H * DV, len);
    GDR_SYNC();
    // Delta block = U - W h = T diag(beta) V - W h  (rows 16w)
    {
      f32x4 aD[NTB], aH[NTB];
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) aD[nt] = aH[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 64 / KW; ++ks)
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt) {
          const frag bv = frag_colk_lds(sV, LDV, 16 * nt, ks * KW);
          aD[nt] = Mma<T>::mma(tbh[ks], bv, aD[nt]);
          if constexpr (SPLIT) aD[nt] = Mma<T>::mma(tbl[ks], bv, aD[nt]);
        }
#pragma unroll
      for (int ks = 0; ks < DK / KW; ++ks) {
        const frag aw = frag_colk_lds(sWT, L64, rw, ks * KW);
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt) aH[nt] = Mma<T>::mma(aw, frag_rowk(sHvk, LDK, 16 * nt, ks * KW), aH[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) store_acc_t2(sDeltaT, sDeltaTl, L64, rw, 16 * nt, aD[nt] - aH[nt]);
    }
    // dQg += dO h^T ; dW -= dDelta h^T ; dT_V += dDelta V^T
#pragma unroll
    for (int ks = 0; ks < DVB / KW; ++ks) {
      const frag ddp = frag_colk_lds(sDDt, L64, rw, ks * KW);
      const frag ddn = Mma<T>::neg(ddp);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) {
        const frag bh = frag_colk_lds(sHvk, LDK, 16 * nt, ks * KW);
        aQ[nt] = Mma<T>::mma(dof[ks], bh, aQ[nt]);
        aW[nt] = Mma<T>::mma(ddn, bh, aW[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aTV[nt] = Mma<T>::mma(ddp, frag_rowk(sV, LDV, 16 * nt, ks * KW), aTV[nt]);
    }
    GDR_SYNC();  // Delta^T complete
    // dKt += Delta dh^T ; dP += dO Delta^T  (Delta split)
#pragma unroll
    for (int ks = 0; ks < DVB / KW; ++ks) {
      const frag ad = frag_colk_lds(sDeltaT, L64, rw, ks * KW);
      frag adl;
      if constexpr (SPLIT) adl = frag_colk_lds(sDeltaTl, L64, rw, ks * KW);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) {
        const frag bdh = frag_colk_lds(sDHvk, LDK, 16 * nt, ks * KW);
        aKt[nt] = Mma<T>::mma(ad, bdh, aKt[nt]);
        if constexpr (SPLIT) aKt[nt] = Mma<T>::mma(adl, bdh, aKt[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        aP[nt] = Mma<T>::mma(dof[ks], frag_colk_lds(sDeltaT, L64, 16 * nt, ks * KW), aP[nt]);
        if constexpr (SPLIT) aP[nt] = Mma<T>::mma(dof[ks], frag_colk_lds(sDeltaTl, L64, 16 * nt, ks * KW), aP[nt]);
      }
    }
    // dVb = T^T dDelta, transposed tiles (lane: row s = rs, 4 columns):
    // dv = beta dVb, dbeta += rowsum(V dVb)
    {
      f32x4 aVb[NTB];
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) aVb[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 64; ks += KW) {
        const frag at = frag_colk_lds(sT, L64, rw, ks);
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt) aVb[nt] = Mma<T>::mma(frag_rowk(sDDt, L64, 16 * nt, ks), at, aVb[nt]);
      }
      const __amdgpu_buffer_rsrc_t rdv = buf_rsrc((T*)a.dv + rowq * DV + dvb, a.dv ? len * H * DV * (int)sizeof(T) : 0);
      const float bs = sb[rs];
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        const f32x4 vv = load4f(sV + rs * LDV + 16 * nt + tc0);
#pragma unroll
        for (int i = 0; i < 4; ++i) rbS += vv[i] * aVb[nt][i];
        buf_store4<T>(rdv, bs * aVb[nt], (rs * H * DV + tc0) * (int)sizeof(T), 16 * nt * (int)sizeof(T));
      }
    }
  }

  // ---------------- phase 2 ----------------
  GDR_SYNC();
  load_rows<T, DK>(sQ, LDK, qp + rowq * DK, (int64_t)H * DK, len);
  load_rows<T, DK>(sK, LDK, kp + rowq * DK, (int64_t)H * DK, len);
  // dW^T -> LDS (aW holds dW rows 16w)
#pragma unroll
  for (int nt = 0; nt < NTK; ++nt) store_acc_t(sdWT, L64, rw, 16 * nt, aW[nt]);
  // gate factor of the 64-wide products at (row r0 + i, column 16 nt +
  // acc_col()): Gam = e^{gamma_r - gamma_s} for s <= r, else 0; per-row and
  // per-column gate values are read from LDS where they are used
  auto gam = [&](int nt, int i) {
    const int r = r0 + i, s = 16 * nt + acc_col();
    const float e = gate_factor<sizeof(T) == 4>(sg, sgl, r, s);
    return (s <= r) ? e : 0.f;
  };
  // dP (scaled, masked) and dQK = dP * Gam -> LDS as (dP * Gam)^T
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 dq4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float dp = (16 * nt + acc_col() <= r0 + i) ? scale * aP[nt][i] : 0.f;
      aP[nt][i] = dp;
      dq4[i] = dp * gam(nt, i);
    }
    store_acc_t(sdQKT, L64, rw, 16 * nt, dq4);
  }
  GDR_SYNC();

  // dgamma from P: rowsum - colsum of dP * P,  P = Q K^T * Gam
  {
    f32x4 aPP[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aPP[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const frag af = frag_rowk(sQ, LDK, rw, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aPP[nt] = Mma<T>::mma(af, frag_rowk(sK, LDK, 16 * nt, ks), aPP[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = aP[nt][i] * aPP[nt][i] * gam(nt, i);
        rg[i] += x;
        cs += x;
      }
      cs = sum4g(cs);
      if (l < 16) sRed[0 * 256 + w * 64 + 16 * nt + l] = cs;
    }
  }
  // dq = e^gamma (scale dO h^T) + (dP * Gam) K ; dgamma += e^gamma rowsum(Q * scale dO h^T)
  {
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) {
      const auto qv = lds_acc(sQ, LDK, rw, 16 * nt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = seg[r0 + i] * scale * aQ[nt][i];
        rg[i] += x * qv[i];
        aQ[nt][i] = x;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const frag af = frag_colk_lds(sdQKT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) aQ[nt] = Mma<T>::mma(af, frag_colk_lds(sK, LDK, 16 * nt, ks), aQ[nt]);
    }
    const __amdgpu_buffer_rsrc_t rdq = buf_rsrc((T*)a.dq + rowq * DK, a.dq ? len * H * DK * (int)sizeof(T) : 0);
    const AccRows ark = acc_rows(H * DK, rw, (int)sizeof(T));
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) buf_store_acc<T>(rdq, ark, 16 * nt, aQ[nt]);
  }
  // dk = E (Delta dh^T) + (dP * Gam)^T Q ; dgamma -= y, gamma_L += sum y
  {
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) {
      const auto kv = lds_acc(sK, LDK, rw, 16 * nt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aKt[nt][i] *= sE[r0 + i];
        const float y = aKt[nt][i] * kv[i];
        rg[i] -= y;
        gLy += y;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const frag af = frag_rowk(sdQKT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) aKt[nt] = Mma<T>::mma(af, frag_colk_lds(sQ, LDK, 16 * nt, ks), aKt[nt]);
    }
  }
  // dKb = T^T dW (rows s = 16w): dk += beta e^gamma dKb, dbeta / dgamma terms
  {
    f32x4 aKb[NTK];
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) aKb[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const frag at = frag_colk_lds(sT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) aKb[nt] = Mma<T>::mma(at, frag_rowk(sdWT, L64, 16 * nt, ks), aKb[nt]);
    }
    float sr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) {
      const auto kv = lds_acc(sK, LDK, rw, 16 * nt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sr[i] += kv[i] * aKb[nt][i];
        aKt[nt][i] += sb[r0 + i] * seg[r0 + i] * aKb[nt][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i;
      rb[i] += seg[r] * sr[i];
      rg[i] += sb[r] * seg[r] * sr[i];
    }
  }
  // dT = dT_V diag(beta) + (dW K^T) diag(beta e^gamma), rows 16w
  f32x4 aT[4];
  {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aT[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const frag af = frag_colk_lds(sdWT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aT[nt] = Mma<T>::mma(af, frag_rowk(sK, LDK, 16 * nt, ks), aT[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * nt + acc_col();
        aT[nt][i] = aTV[nt][i] * sb[s] + aT[nt][i] * sb[s] * seg[s];
      }
  }
  GDR_SYNC();  // all reads of sQ, sdQKT, sdWT done
  T* sTT = sQ;      // dT^T (s, r)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) store_acc_t(sTT, L64, rw, 16 * nt, aT[nt]);
  GDR_SYNC();
  // Y = T^T dT (rows a = 16w) -> LDS as Y^T
  {
    f32x4 aY[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aY[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const frag at = frag_colk_lds(sT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aY[nt] = Mma<T>::mma(at, frag_rowk(sTT, L64, 16 * nt, ks), aY[nt]);
    }
    T* sYT = sdQKT;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) store_acc_t(sYT, L64, rw, 16 * nt, aY[nt]);
  }
  GDR_SYNC();
  // dA = -(Y T^T) strictly lower; K K^T; dbeta, dgamma terms; G -> LDS as G^T
  {
    const T* sYT = sdQKT;
    f32x4 aA[4], aKK[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aA[nt] = aKK[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const frag ay = frag_colk_lds(sYT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aA[nt] = Mma<T>::mma(ay, frag_rowk(sT, L64, 16 * nt, ks), aA[nt]);
    }
#pragma unroll
    for (int ks = 0; ks < DK; ks += KW) {
      const frag ak = frag_rowk(sK, LDK, rw, ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aKK[nt] = Mma<T>::mma(ak, frag_rowk(sK, LDK, 16 * nt, ks), aKK[nt]);
    }
    T* sGT = sdWT;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 G;
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // strictly lower part: Gam without its diagonal
        const int r = r0 + i, s = 16 * nt + acc_col();
        float gv = 0.f;
        if (s < r) {
          const float Gm = gate_factor<sizeof(T) == 4>(sg, sgl, r, s);
          const float dA = -aA[nt][i];
          rb[i] += dA * aKK[nt][i] * Gm;
          const float X = dA * sb[r] * aKK[nt][i] * Gm;
          rg[i] += X;
          cs += X;
          gv = dA * sb[r] * Gm;
        }
        G[i] = gv;
      }
      cs = sum4g(cs);
      if (l < 16) sRed[1 * 256 + w * 64 + 16 * nt + l] = cs;
      store_acc_t(sGT, L64, rw, 16 * nt, G);
    }
  }
  // per-wave gamma_L partials (lanes 0..63 summed)
  {
    const float xh = sum4g(sum16(gLh));
    const float xy = sum4g(sum16(gLy));
    if (l == 0) {
      sMisc[w] = xh;
      sMisc[4 + w] = xy;
    }
  }
  GDR_SYNC();
  // dk += G K + G^T K, write dk
  {
    const T* sGT = sdWT;
#pragma unroll
    for (int ks = 0; ks < 64; ks += KW) {
      const frag a1 = frag_colk_lds(sGT, L64, rw, ks);
      const frag a2 = frag_rowk(sGT, L64, rw, ks);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) {
        const frag bk = frag_colk_lds(sK, LDK, 16 * nt, ks);
        aKt[nt] = Mma<T>::mma(a1, bk, aKt[nt]);
        aKt[nt] = Mma<T>::mma(a2, bk, aKt[nt]);
      }
    }
    const __amdgpu_buffer_rsrc_t rdk = buf_rsrc((T*)a.dk + rowq * DK, a.dk ? len * H * DK * (int)sizeof(T) : 0);
    const AccRows ark = acc_rows(H * DK, rw, (int)sizeof(T));
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) buf_store_acc<T>(rdk, ark, 16 * nt, aKt[nt]);
  }
  // row sums -> LDS (one writer per row), then dbeta, dgamma -> dg.  The
  // accumulator-tile terms of a row are spread over the 16 lanes sharing
  // l >> 4, the transposed-tile terms over the 4 lanes sharing l & 15.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rg[i] = sum16(rg[i]);
    rb[i] = sum16(rb[i]);
  }
  rbS = sum4g(rbS);
  GDR_SYNC();
  float* sRG = (float*)sQ;        // phase-2 LDS is free now
  float* sRB = sRG + 64;
  float* sRB2 = sRB + 64;
  if ((l & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sRG[r0 + i] = rg[i];
      sRB[r0 + i] = rb[i];
    }
  }
  if (l < 16) {
    sRB2[rs] = rbS;
  }
  GDR_SYNC();
  if (w == 0) {
    float dgam = sRG[l] -
                 (sRed[0 * 256 + 0 * 64 + l] + sRed[0 * 256 + 1 * 64 + l] + sRed[0 * 256 + 2 * 64 + l] +
                  sRed[0 * 256 + 3 * 64 + l]) -
                 (sRed[1 * 256 + 0 * 64 + l] + sRed[1 * 256 + 1 * 64 + l] + sRed[1 * 256 + 2 * 64 + l] +
                  sRed[1 * 256 + 3 * 64 + l]);
    if (l == 63) {
      // gamma_L terms: e^{gamma_L} <dh, h> and sum_r E_r rowsum(K * Delta dh^T)
      dgam += seg[63] * (sMisc[0] + sMisc[1] + sMisc[2] + sMisc[3]) +
              (sMisc[4] + sMisc[5] + sMisc[6] + sMisc[7]);
    }
    const float dgv = wave_suffix_scan(dgam);
    if (l < len) {
      if (a.dg) a.dg[(int64_t)(t0 + l) * H + h] = dgv;
      if (a.dbeta) a.dbeta[(int64_t)(t0 + l) * H + h] = sRB[l] + sRB2[l];
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int DK, int MODE>
static hipError_t launch_scan_bwd_t(ScanBwdArgs a, int dvt, hipStream_t st) {
  const int units = a.geo.N * a.geo.cp * a.geo.H;
  a.ntiles = ((MODE == 0 ? DK : 0) + a.DV) / dvt;
  const int grid = 8 * ((units + 7) / 8) * a.ntiles;
  if (units == 0) return hipSuccess;
  if (dvt == 16) hipLaunchKernelGGL((k_scan_bwd<T, DK, 16, MODE>), dim3(grid), dim3(256), 0, st, a);
  else if constexpr (sizeof(T) == 2) {
    if (dvt == 32) hipLaunchKernelGGL((k_scan_bwd<T, DK, 32, MODE>), dim3(grid), dim3(256), 0, st, a);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_scan_bwd_m(const ScanBwdArgs& a, int dvt, int mode, hipStream_t st) {
  return mode == 0 ? launch_scan_bwd_t<T, DK, 0>(a, dvt, st) : launch_scan_bwd_t<T, DK, 1>(a, dvt, st);
}

hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool f32, int DK, int dvt, int mode, hipStream_t st) {
  if (f32) return DK == 64 ? launch_scan_bwd_m<float, 64>(a, dvt, mode, st) : launch_scan_bwd_m<float, 128>(a, dvt, mode, st);
  return DK == 64 ? launch_scan_bwd_m<bf16, 64>(a, dvt, mode, st) : launch_scan_bwd_m<bf16, 128>(a, dvt, mode, st);
}

template <typename T, int DK>
static size_t grad_smem() {
  constexpr int P = pad_of<T>();
  constexpr int LDK = DK + P, L64 = 64 + P, DVB = GRAD_DVB, LDV = DVB + P;
  constexpr int PH1 = (2 * DVB * LDK + 3 * DVB * L64 + 64 * LDV + DK * L64) * (int)sizeof(T);
  constexpr int PH2 = (2 * 64 * LDK + DK * L64 + 64 * L64) * (int)sizeof(T);
  return 64 * L64 * sizeof(T) + (5 * 64 + 2 * 4 * 64 + 8) * 4 + cmax(PH1, PH2);
}

template <typename T, typename HS, int DK>
static hipError_t launch_grad_t(const GradArgs& a, hipStream_t st) {
  const size_t sm = grad_smem<T, DK>();
  hipError_t e = hipFuncSetAttribute((const void*)k_grad<T, HS, DK>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_grad<T, HS, DK>), dim3(a.geo.nchunks, a.geo.H), dim3(256), sm, st, a);
  return hipGetLastError();
}

hipError_t launch_grad(const GradArgs& a, bool f32, int hs_dtype, int DK, hipStream_t st) {
  if (f32) return DK == 64 ? launch_grad_t<float, float, 64>(a, st) : launch_grad_t<float, float, 128>(a, st);
  if (hs_dtype == GDR_F32) return DK == 64 ? launch_grad_t<bf16, float, 64>(a, st) : launch_grad_t<bf16, float, 128>(a, st);
  if (hs_dtype == GDR_F16) return DK == 64 ? launch_grad_t<bf16, f16, 64>(a, st) : launch_grad_t<bf16, f16, 128>(a, st);
  return DK == 64 ? launch_grad_t<bf16, bf16, 64>(a, st) : launch_grad_t<bf16, bf16, 128>(a, st);
}

#ifdef GDR_DEBUG_DELAY
// the race-test build: this file's copy of the barrier-delay settings
hipError_t debug_set_delay_bwd(const DelayCfg& c) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_delay), &c, sizeof(c));
}
#endif

}  // namespace gdr
