/*
 * gdr_oracle.c -- fp64 CPU oracle for the gated delta rule (GDR).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that the tests, the smoke check and the
 * benchmark's CPU-baseline leg can check the HIP library against a plain,
 * slow, obviously-correct computation.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * What it computes.  The pages name the operator -- "the chunked gated delta
 * rule" and its fused backward fused_gdr_bwd (FlashQLA PR #34, "SM120/121 :
 * Add support for fused backward kernel", section "Summary") -- with features
 * fixed-length and variable-length inputs, KV/VK state layouts and initial /
 * final states (same page, section "Current status").  The pages never print
 * the recurrence; this oracle uses the standard gated delta rule, per
 * (sequence, head), with state S in R^{DV x DK} ("VK" form):
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t,          S_0 = h0 (zero if absent), h_T = S_T.
 *
 * It is evaluated token by token in the equivalent "delta" form
 *     (R1) St  = a_t S_{t-1},  a_t = exp(g_t)
 *     (R2) p   = St k_t
 *     (R3) d   = beta_t (v_t - p)
 *     (R4) S_t = St + d k_t^T
 *     (R5) o_t = scale S_t q_t
 * which is the recurrence above with the product expanded (a_t S (I - b k k^T)
 * + b v k^T = a_t S + b (v - a_t S k) k^T).  The chunked algorithm computes
 * exactly this result in exact arithmetic, so no step of it is modelled here.
 *
 * The backward is reverse-mode differentiation of R1-R5, derived by hand:
 *     (O1) dS += scale do_t q_t^T        (O2)  dq_t  = scale S_t^T do_t
 *     (O3) dd  = dS k_t                  (O4)  dk_t  = dS^T d
 *     (O5) dbeta_t = dd . (v_t - p)      (O6)  dv_t  = beta_t dd
 *     (O7) dp  = -beta_t dd              (O8)  dSt   = dS + dp k_t^T
 *     (O9) dk_t += St^T dp               (O10) dg_t  = <dSt, St>_F
 *     (O11) dS = a_t dSt                 (O12) dh0   = dS after t = 1.
 * dS starts at dh_T (zero if absent).  The reverse sweep recomputes the
 * states of each 64-token segment from a checkpoint taken in a forward sweep,
 * so memory is O(T/64 * DV * DK) per (sequence, head).
 *
 * Memory layout (all fp64, all contiguous):
 *   tokens are packed along one dimension of length Ttot; sequence n occupies
 *   tokens [start[n], start[n] + len[n]).  q,k: [Ttot][H][DK]; v,o,do:
 *   [Ttot][H][DV]; beta,g: [Ttot][H]; states h0,hT,dhT,dh0: [N][H][DV][DK]
 *   (VK form; the caller transposes for the KV form -- a pure relayout).
 *
 * Parallelism: OpenMP over (sequence, head) pairs, which are independent.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CKPT 64

typedef struct {
  int64_t n, hd;
} pair_t;

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int gdr_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One token of the forward recurrence (R1-R5).  S: DV x DK, updated in place.
 * p (DV) and d (DV) are scratch; o_t (DV) may be NULL. */
static void token_forward(int DK, int DV, double scale, double* S, const double* qt,
                          const double* kt, const double* vt, double bt, double gt, double* p,
                          double* d, double* ot) {
  const double a = exp(gt);
  for (int i = 0; i < DV; ++i) {
    double* Si = S + (size_t)i * DK;
    double acc = 0.0;
    for (int j = 0; j < DK; ++j) {
      Si[j] *= a;                 /* R1 */
      acc += Si[j] * kt[j];       /* R2 */
    }
    p[i] = acc;
    d[i] = bt * (vt[i] - acc);    /* R3 */
    for (int j = 0; j < DK; ++j) Si[j] += d[i] * kt[j]; /* R4 */
  }
  if (ot) {
    for (int i = 0; i < DV; ++i) {
      const double* Si = S + (size_t)i * DK;
      double acc = 0.0;
      for (int j = 0; j < DK; ++j) acc += Si[j] * qt[j];
      ot[i] = scale * acc;        /* R5 */
    }
  }
}

/* Forward: o and (optionally) h_T.  Returns 0 on success, 1 on allocation
 * failure. */
int gdr_oracle_fwd(int N, const int64_t* start, const int64_t* len, int H, int DK, int DV,
                   double scale, const double* q, const double* k, const double* v,
                   const double* beta, const double* g, const double* h0, double* o,
                   double* hT, int nthreads) {
  set_threads(nthreads);
  const int64_t npairs = (int64_t)N * H;
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
  for (int64_t pi = 0; pi < npairs; ++pi) {
    const int64_t n = pi / H, hd = pi % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)DV * DK);
    double* p = (double*)malloc(sizeof(double) * (size_t)DV);
    double* d = (double*)malloc(sizeof(double) * (size_t)DV);
    if (!S || !p || !d) {
      free(S); free(p); free(d);
      fail |= 1;
      continue;
    }
    const size_t soff = ((size_t)n * H + hd) * DV * DK;
    if (h0) memcpy(S, h0 + soff, sizeof(double) * (size_t)DV * DK);
    else memset(S, 0, sizeof(double) * (size_t)DV * DK);
    for (int64_t t = start[n]; t < start[n] + len[n]; ++t) {
      const size_t th = (size_t)t * H + hd;
      token_forward(DK, DV, scale, S, q + th * DK, k + th * DK, v + th * DV, beta[th], g[th], p,
                    d, o + th * DV);
    }
    if (hT) memcpy(hT + soff, S, sizeof(double) * (size_t)DV * DK);
    free(S); free(p); free(d);
  }
  return fail;
}

/* Backward (O1-O12).  Any of dq,dk,dv,dbeta,dg may not be NULL; dh0 may be
 * NULL (not written); dhT may be NULL (zero). */
int gdr_oracle_bwd(int N, const int64_t* start, const int64_t* len, int H, int DK, int DV,
                   double scale, const double* q, const double* k, const double* v,
                   const double* beta, const double* g, const double* h0, const double* dO,
                   const double* dhT, double* dq, double* dk, double* dv, double* dbeta,
                   double* dg, double* dh0, int nthreads) {
  set_threads(nthreads);
  const int64_t npairs = (int64_t)N * H;
  const size_t SS = (size_t)DV * DK;
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
  for (int64_t pi = 0; pi < npairs; ++pi) {
    const int64_t n = pi / H, hd = pi % H;
    const int64_t T0 = start[n], L = len[n];
    const int64_t nseg = (L + ORACLE_CKPT - 1) / ORACLE_CKPT;
    const size_t soff = ((size_t)n * H + hd) * SS;
    /* ckpt[m] = state before token m*CKPT of this sequence. */
    double* ckpt = (double*)malloc(sizeof(double) * SS * (size_t)(nseg > 0 ? nseg : 1));
    /* sprev[j] = state before the j-th token of the current segment. */
    double* sprev = (double*)malloc(sizeof(double) * SS * (ORACLE_CKPT + 1));
    double* dS = (double*)malloc(sizeof(double) * SS);
    double* St = (double*)malloc(sizeof(double) * SS);
    double* p = (double*)malloc(sizeof(double) * DV);
    double* d = (double*)malloc(sizeof(double) * DV);
    double* dd = (double*)malloc(sizeof(double) * DV);
    double* dp = (double*)malloc(sizeof(double) * DV);
    if (!ckpt || !sprev || !dS || !St || !p || !d || !dd || !dp) {
      free(ckpt); free(sprev); free(dS); free(St); free(p); free(d); free(dd); free(dp);
      fail |= 1;
      continue;
    }
    /* forward sweep, checkpointing */
    double* S = sprev; /* borrow as running state */
    if (h0) memcpy(S, h0 + soff, sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (int64_t t = 0; t < L; ++t) {
      if (t % ORACLE_CKPT == 0) memcpy(ckpt + (size_t)(t / ORACLE_CKPT) * SS, S, sizeof(double) * SS);
      const size_t th = (size_t)(T0 + t) * H + hd;
      token_forward(DK, DV, scale, S, NULL, k + th * DK, v + th * DV, beta[th], g[th], p, d, NULL);
    }
    if (dhT) memcpy(dS, dhT + soff, sizeof(double) * SS);
    else memset(dS, 0, sizeof(double) * SS);
    /* reverse sweep, segment by segment */
    for (int64_t m = nseg - 1; m >= 0; --m) {
      const int64_t s0 = m * ORACLE_CKPT;
      const int64_t s1 = (s0 + ORACLE_CKPT < L) ? s0 + ORACLE_CKPT : L;
      memcpy(sprev, ckpt + (size_t)m * SS, sizeof(double) * SS);
      for (int64_t t = s0; t < s1; ++t) {
        const size_t th = (size_t)(T0 + t) * H + hd;
        double* nxt = sprev + (size_t)(t - s0 + 1) * SS;
        memcpy(nxt, sprev + (size_t)(t - s0) * SS, sizeof(double) * SS);
        token_forward(DK, DV, scale, nxt, NULL, k + th * DK, v + th * DV, beta[th], g[th], p, d,
                      NULL);
      }
      for (int64_t t = s1 - 1; t >= s0; --t) {
        const size_t th = (size_t)(T0 + t) * H + hd;
        const double* qt = q + th * DK;
        const double* kt = k + th * DK;
        const double* vt = v + th * DV;
        const double* dot = dO + th * DV;
        const double bt = beta[th];
        const double a = exp(g[th]);
        const double* Sprev = sprev + (size_t)(t - s0) * SS;   /* S_{t-1} */
        const double* Snow = sprev + (size_t)(t - s0 + 1) * SS; /* S_t */
        /* St = a S_{t-1}; p = St k; d = beta (v - p) */
        for (size_t e = 0; e < SS; ++e) St[e] = a * Sprev[e];
        for (int i = 0; i < DV; ++i) {
          double acc = 0.0;
          for (int j = 0; j < DK; ++j) acc += St[(size_t)i * DK + j] * kt[j];
          p[i] = acc;
          d[i] = bt * (vt[i] - acc);
        }
        /* O1 */
        for (int i = 0; i < DV; ++i)
          for (int j = 0; j < DK; ++j) dS[(size_t)i * DK + j] += scale * dot[i] * qt[j];
        /* O2 */
        for (int j = 0; j < DK; ++j) {
          double acc = 0.0;
          for (int i = 0; i < DV; ++i) acc += Snow[(size_t)i * DK + j] * dot[i];
          dq[th * DK + j] = scale * acc;
        }
        /* O3 */
        for (int i = 0; i < DV; ++i) {
          double acc = 0.0;
          for (int j = 0; j < DK; ++j) acc += dS[(size_t)i * DK + j] * kt[j];
          dd[i] = acc;
        }
        /* O4 */
        for (int j = 0; j < DK; ++j) {
          double acc = 0.0;
          for (int i = 0; i < DV; ++i) acc += dS[(size_t)i * DK + j] * d[i];
          dk[th * DK + j] = acc;
        }
        /* O5, O6, O7 */
        double db = 0.0;
        for (int i = 0; i < DV; ++i) {
          db += dd[i] * (vt[i] - p[i]);
          dv[th * DV + i] = bt * dd[i];
          dp[i] = -bt * dd[i];
        }
        dbeta[th] = db;
        /* O8: dSt = dS + dp k^T (in place in dS) */
        for (int i = 0; i < DV; ++i)
          for (int j = 0; j < DK; ++j) dS[(size_t)i * DK + j] += dp[i] * kt[j];
        /* O9 */
        for (int j = 0; j < DK; ++j) {
          double acc = 0.0;
          for (int i = 0; i < DV; ++i) acc += St[(size_t)i * DK + j] * dp[i];
          dk[th * DK + j] += acc;
        }
        /* O10 */
        double gg = 0.0;
        for (size_t e = 0; e < SS; ++e) gg += dS[e] * St[e];
        dg[th] = gg;
        /* O11 */
        for (size_t e = 0; e < SS; ++e) dS[e] *= a;
      }
    }
    if (dh0) memcpy(dh0 + soff, dS, sizeof(double) * SS); /* O12 */
    free(ckpt); free(sprev); free(dS); free(St); free(p); free(d); free(dd); free(dp);
  }
  return fail;
}
