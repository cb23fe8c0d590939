// gdr_api.cpp -- host side of libgdr: argument validation, workspace layout,
// launch planning.  Implements the C ABI declared in include/libgdr.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "gdr_host.h"
#include "gdr_kernels.h"

namespace {

thread_local char g_err[512] = "";
thread_local bool g_timed = false;
thread_local hipEvent_t g_events[2 * GDR_NUM_KERNELS];

void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

size_t elt(int dtype) { return dtype == GDR_F32 ? 4 : 2; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

gdr_status check_problem(const gdr_problem* p) {
  if (!p) { set_err("problem is NULL"); return GDR_ERR_INVALID_ARG; }
  if (p->batch < 1) { set_err("batch must be >= 1 (got %d)", p->batch); return GDR_ERR_INVALID_ARG; }
  if (p->seqlen < 0) { set_err("seqlen must be >= 0 (got %d)", p->seqlen); return GDR_ERR_INVALID_ARG; }
  if (p->heads < 1) { set_err("heads must be >= 1 (got %d)", p->heads); return GDR_ERR_INVALID_ARG; }
  if (p->varlen != 0 && p->varlen != 1) { set_err("varlen must be 0 or 1"); return GDR_ERR_INVALID_ARG; }
  if (p->varlen) {
    if (p->batch != 1) { set_err("packed (varlen) batches need batch == 1 (got %d)", p->batch); return GDR_ERR_INVALID_ARG; }
    if (p->num_seqs < 1) { set_err("num_seqs must be >= 1 (got %d)", p->num_seqs); return GDR_ERR_INVALID_ARG; }
    if (p->num_seqs > GDR_MAX_SEQS) {
      set_err("num_seqs %d exceeds the supported maximum %d", p->num_seqs, GDR_MAX_SEQS);
      return GDR_ERR_UNSUPPORTED;
    }
  } else if (p->num_seqs != p->batch) {
    set_err("num_seqs (%d) must equal batch (%d) for fixed-length batches", p->num_seqs, p->batch);
    return GDR_ERR_INVALID_ARG;
  }
  if (p->chunk != 64) { set_err("chunk must be 64 (got %d)", p->chunk); return GDR_ERR_UNSUPPORTED; }
  if (p->dk != 64 && p->dk != 128) { set_err("dk must be 64 or 128 (got %d)", p->dk); return GDR_ERR_UNSUPPORTED; }
  if (p->dv < 64 || p->dv > 512 || p->dv % 64 != 0) {
    set_err("dv must be a multiple of 64 in [64, 512] (got %d)", p->dv);
    return GDR_ERR_UNSUPPORTED;
  }
  if (p->io_dtype != GDR_F32 && p->io_dtype != GDR_BF16) { set_err("io_dtype must be GDR_F32 or GDR_BF16"); return GDR_ERR_UNSUPPORTED; }
  if (p->h_store_dtype != GDR_F32 && p->h_store_dtype != GDR_F16 && p->h_store_dtype != GDR_BF16) {
    set_err("h_store_dtype must be GDR_F32, GDR_F16 or GDR_BF16");
    return GDR_ERR_INVALID_ARG;
  }
  if (p->io_dtype == GDR_F32 && p->h_store_dtype != GDR_F32) {
    set_err("fp32 inputs need fp32 state snapshots");
    return GDR_ERR_UNSUPPORTED;
  }
  if (p->layout != GDR_LAYOUT_KV && p->layout != GDR_LAYOUT_VK) { set_err("layout must be GDR_LAYOUT_KV or GDR_LAYOUT_VK"); return GDR_ERR_INVALID_ARG; }
  if (p->cp_segments < 1) { set_err("cp_segments must be >= 1 (got %d)", p->cp_segments); return GDR_ERR_INVALID_ARG; }
  if (p->cp_segments > 1024) { set_err("cp_segments must be <= 1024 (got %d)", p->cp_segments); return GDR_ERR_UNSUPPORTED; }
  const double tokens = (double)p->batch * p->seqlen;
  const int dmax = p->dv > p->dk ? p->dv : p->dk;
  if (tokens * p->heads * dmax > 4.0e12) { set_err("problem too large"); return GDR_ERR_UNSUPPORTED; }
  // the kernels address one chunk (64 token rows of H heads) of a [B, T, H, D]
  // tensor through a raw buffer whose range and offsets are 32-bit byte counts
  if (64.0 * p->heads * dmax * (double)elt(p->io_dtype) > 2147483647.0) {
    set_err("64 x heads x max(dk, dv) x element size must stay below 2^31 bytes (heads %d, d %d)", p->heads, dmax);
    return GDR_ERR_UNSUPPORTED;
  }
  return GDR_OK;
}

struct Plan {
  int N = 0, NCb = 0, ncps = 0;
  bool f32 = false;
  size_t esz = 2, hsz = 4;
  size_t seq_chunk = 0, chunk_seq = 0, gam = 0, gaml = 0, Wf = 0, KtTf = 0, Ua = 0, hs = 0, Qf = 0, Pf = 0, Pfl = 0;
  size_t Tm = 0, WTf = 0, Kf = 0, dDl = 0, Z = 0, dhs = 0, dD = 0;
  size_t summ = 0, hst = 0;   // CP segment summaries and hand-off states
  size_t total = 0;
};

// mode 0: forward, 1: backward.  need_hs: the snapshots live in the
// workspace (forward without h_saved, backward recomputing them).
Plan make_plan(const gdr_problem* p, int mode, bool need_hs) {
  Plan pl;
  pl.N = p->varlen ? p->num_seqs : p->batch;
  pl.f32 = p->io_dtype == GDR_F32;
  pl.esz = elt(p->io_dtype);
  pl.hsz = elt(p->h_store_dtype);
  if (p->varlen) {
    pl.NCb = (p->seqlen + 63) / 64 + pl.N;
    pl.ncps = 0;
  } else {
    pl.ncps = (p->seqlen + 63) / 64;
    pl.NCb = p->batch * pl.ncps;
  }
  const size_t ch = (size_t)pl.NCb * p->heads;
  const size_t DK = p->dk, DV = p->dv, e = pl.esz;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  if (p->varlen) {
    pl.seq_chunk = take(sizeof(int) * (pl.N + 1));
    pl.chunk_seq = take(sizeof(int) * (size_t)pl.NCb);
  }
  pl.gam = take(ch * GSTRIDE * 4);
  if (mode == 0 || need_hs) {   // the backward's gradient kernel needs neither
    pl.Wf = take(ch * 64 * DK * e);
    pl.Ua = take(ch * 64 * DV * 4);
  }
  if (need_hs) {
    pl.hs = take(ch * DV * DK * pl.hsz);
    pl.KtTf = take(ch * DK * 64 * e);
  }
  if (mode == 0) {
    if (!need_hs) pl.KtTf = take(ch * DK * 64 * e);
    pl.Qf = take(ch * 64 * DK * e);
    pl.Pf = take(ch * 64 * 64 * e);
    if (!pl.f32) pl.Pfl = take(ch * 64 * 64 * e);
  } else {
    pl.Tm = take(ch * 64 * 64 * 4);
    pl.WTf = take(ch * DK * 64 * e);
    pl.Kf = take(ch * 64 * DK * e);
    pl.dDl = take(ch * 64 * DV * 4);
    pl.Z = take(ch * DK * DV * 4);
    pl.dhs = take(ch * DK * DV * e);
    pl.dD = take(ch * 64 * DV * e);
  }
  if (p->cp_segments > 1) {
    const size_t units = (size_t)p->cp_segments * pl.N * p->heads;
    pl.summ = take(units * DK * (DK + DV) * 4);
    pl.hst = take(units * DK * DV * 4);
  }
  // the lo part of gamma goes last: placed beside the gate blocks it moved
  // every later buffer and measurably slowed the forward scan (4-5 us at
  // B=2, T=4096, H=16, D=128), which reads them all in step
  pl.gaml = take(ch * 64 * 4);
  pl.total = o + 256;  // slack for base alignment
  return pl;
}

bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15) != 0; }

gdr::Geo make_geo(const gdr_problem* p, const Plan& pl, const int32_t* cu, char* ws) {
  gdr::Geo g;
  g.H = p->heads;
  g.N = pl.N;
  g.T_fixed = p->varlen ? 0 : p->seqlen;
  g.nc_per_seq = pl.ncps;
  g.nchunks = pl.NCb;
  g.T_total = p->seqlen;
  g.cu = p->varlen ? cu : nullptr;
  g.seq_chunk = p->varlen ? (const int*)(ws + pl.seq_chunk) : nullptr;
  g.chunk_seq = p->varlen ? (const int*)(ws + pl.chunk_seq) : nullptr;
  g.cp = p->cp_segments;
  return g;
}

// Column tile of the serial scans.  A wider tile reads each chunk operand
// once for more columns, a narrower one gives more workgroups: take the
// widest that still gives one workgroup per compute unit (256 in all), among
// the widths measured faster (64 for the forward output scan, 32 for the
// others: at 64 their rings no longer fit two waves per SIMD).  The fp32
// path always uses 16 (its operand fragments are 8x larger per k).
int pick_dvt(long units, int cols, bool f32, bool out = false) {
  if (f32) return 16;
  if (out && cols % 64 == 0 && units * (cols / 64) >= 256) return 64;
  return units * (cols / 32) >= 256 ? 32 : 16;
}

char* align_ws(void* ws) { return (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255); }

#define GDR_TRY(expr)                                                        \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ != hipSuccess) {                                                  \
      set_err("%s failed: %s", #expr, hipGetErrorString(e_));                \
      return GDR_ERR_HIP;                                                    \
    }                                                                        \
  } while (0)

// Launch with optional start/stop events (diagnostic timers of this thread).
#define GDR_LAUNCH(kid, stream, expr)                                              \
  do {                                                                            \
    hipEvent_t st_ = g_timed ? g_events[2 * (kid)] : nullptr;                     \
    hipEvent_t sp_ = g_timed ? g_events[2 * (kid) + 1] : nullptr;                 \
    if (st_) GDR_TRY(hipEventRecord(st_, stream));                                \
    GDR_TRY(expr);                                                                \
    if (sp_) GDR_TRY(hipEventRecord(sp_, stream));                                \
  } while (0)

}  // namespace

namespace gdr {

void set_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }

size_t fwd_workspace_bytes(const gdr_problem* p) { return make_plan(p, 0, false).total; }

// The forward proper, on a caller-provided workspace (gdr_chunk_fwd) or the
// library's static one (gdr_chunk_fwd_noalloc).
gdr_status chunk_fwd_impl(const gdr_problem* p, const void* q, const void* k, const void* v,
                          const float* beta, const float* g, const int32_t* cu_seqlens,
                          const float* h0, void* o, float* hT, void* h_saved, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  const bool tokens = (int64_t)p->batch * p->seqlen > 0;
  if (tokens && (!q || !k || !v || !beta || !g || !o)) { set_err("q, k, v, beta, g and o are required"); return GDR_ERR_INVALID_ARG; }
  if ((p->varlen != 0) != (cu_seqlens != nullptr)) { set_err("cu_seqlens must be given exactly when varlen is 1"); return GDR_ERR_INVALID_ARG; }
  const void* ptrs[] = {q, k, v, beta, g, o, h0, hT, h_saved, cu_seqlens};
  for (const void* ptr : ptrs)
    if (ptr && misaligned(ptr)) { set_err("all buffers must be 16-byte aligned"); return GDR_ERR_INVALID_ARG; }
  const Plan pl = make_plan(p, 0, false);   // snapshots go to h_saved or nowhere
  if (!workspace || workspace_bytes < pl.total) {
    set_err("workspace of %zu bytes needed (got %zu)", pl.total, workspace ? workspace_bytes : (size_t)0);
    return GDR_ERR_WORKSPACE;
  }
  char* ws = align_ws(workspace);
  hipStream_t s = (hipStream_t)stream;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->dk);
  gdr::Geo geo = make_geo(p, pl, cu_seqlens, ws);
  void* hs = h_saved;

  if (p->varlen)
    GDR_LAUNCH(GDR_KERNEL_PLAN, s, gdr::launch_plan(cu_seqlens, pl.N, p->seqlen, pl.NCb, (int*)(ws + pl.seq_chunk), (int*)(ws + pl.chunk_seq), s));
  if (pl.NCb > 0) {
    gdr::WyArgs wa{};
    wa.geo = geo; wa.DV = p->dv; wa.scale = scale;
    wa.q = q; wa.k = k; wa.v = v; wa.beta = beta; wa.g = g;
    wa.gam = (float*)(ws + pl.gam); wa.gaml = (float*)(ws + pl.gaml); wa.Wf = ws + pl.Wf; wa.KtTf = ws + pl.KtTf; wa.Ua = (float*)(ws + pl.Ua);
    wa.Qf = ws + pl.Qf; wa.Pf = ws + pl.Pf; wa.Pfl = pl.f32 ? nullptr : (void*)(ws + pl.Pfl);
    GDR_LAUNCH(GDR_KERNEL_WY, s, gdr::launch_wy(wa, pl.f32, p->dk, false, s));
  }
  gdr::ScanFwdArgs sa{};
  sa.geo = geo; sa.DV = p->dv; sa.layout = p->layout; sa.scale = scale; sa.h0 = h0; sa.hT = hT;
  sa.gam = (const float*)(ws + pl.gam); sa.Wf = ws + pl.Wf; sa.KtTf = ws + pl.KtTf; sa.Ua = (const float*)(ws + pl.Ua);
  sa.Qf = ws + pl.Qf; sa.Pf = ws + pl.Pf; sa.Pfl = ws + pl.Pfl; sa.o = o; sa.hs = hs;
  const long units = (long)pl.N * p->cp_segments * p->heads;
  if (p->cp_segments > 1) {
    sa.summ = (float*)(ws + pl.summ); sa.hstart = (const float*)(ws + pl.hst);
    GDR_LAUNCH(GDR_KERNEL_CP_SCAN_FWD, s, gdr::launch_scan_fwd(sa, pl.f32, p->h_store_dtype, p->dk, pick_dvt(units, p->dk + p->dv, pl.f32), 0, s));
    gdr::CpChainArgs ca{geo, p->dk, p->dv, p->layout, 0, h0, (const float*)(ws + pl.summ), (float*)(ws + pl.hst)};
    GDR_LAUNCH(GDR_KERNEL_CP_CHAIN_FWD, s, gdr::launch_cp_chain(ca, s));
  }
  // mode 2 writes the snapshots to h_saved; mode 3 keeps none
  GDR_LAUNCH(GDR_KERNEL_SCAN_FWD, s, gdr::launch_scan_fwd(sa, pl.f32, p->h_store_dtype, p->dk, pick_dvt(units, p->dv, pl.f32, true), h_saved ? 2 : 3, s));
  return GDR_OK;
}

}  // namespace gdr

extern "C" {

gdr_status gdr_check(const gdr_problem* p) {
  g_err[0] = 0;
  return check_problem(p);
}

size_t gdr_fwd_workspace_bytes(const gdr_problem* p) {
  if (check_problem(p) != GDR_OK) return 0;
  return make_plan(p, 0, false).total;
}

size_t gdr_bwd_workspace_bytes(const gdr_problem* p, int have_h_saved) {
  if (check_problem(p) != GDR_OK) return 0;
  return make_plan(p, 1, !have_h_saved).total;
}

size_t gdr_h_saved_bytes(const gdr_problem* p) {
  if (check_problem(p) != GDR_OK) return 0;
  Plan pl = make_plan(p, 0, false);
  return (size_t)pl.NCb * p->heads * p->dv * p->dk * pl.hsz;
}

gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, const int32_t* cu_seqlens,
                         const float* h0, void* o, float* hT, void* h_saved, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return gdr::chunk_fwd_impl(p, q, k, v, beta, g, cu_seqlens, h0, o, hT, h_saved, workspace, workspace_bytes,
                             stream);
}

gdr_status gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, const int32_t* cu_seqlens,
                         const float* h0, const void* h_saved, const void* dO, const float* dhT,
                         void* dq, void* dk, void* dv, float* dbeta, float* dg, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  const bool tokens = (int64_t)p->batch * p->seqlen > 0;
  if (tokens && (!q || !k || !v || !beta || !g || !dO)) {
    set_err("q, k, v, beta, g and dO are required");
    return GDR_ERR_INVALID_ARG;
  }
  if ((p->varlen != 0) != (cu_seqlens != nullptr)) { set_err("cu_seqlens must be given exactly when varlen is 1"); return GDR_ERR_INVALID_ARG; }
  const void* ptrs[] = {q, k, v, beta, g, dO, dq, dk, dv, dbeta, dg, h0, h_saved, dhT, dh0, cu_seqlens};
  for (const void* ptr : ptrs)
    if (ptr && misaligned(ptr)) { set_err("all buffers must be 16-byte aligned"); return GDR_ERR_INVALID_ARG; }
  const Plan pl = make_plan(p, 1, h_saved == nullptr);
  if (!workspace || workspace_bytes < pl.total) {
    set_err("workspace of %zu bytes needed (got %zu)", pl.total, workspace ? workspace_bytes : (size_t)0);
    return GDR_ERR_WORKSPACE;
  }
  char* ws = align_ws(workspace);
  hipStream_t s = (hipStream_t)stream;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->dk);
  gdr::Geo geo = make_geo(p, pl, cu_seqlens, ws);
  const void* hs = h_saved ? h_saved : (const void*)(ws + pl.hs);
  const long units = (long)pl.N * p->cp_segments * p->heads;
  const int dvt = pick_dvt(units, p->dv, pl.f32);
  const int dvt_cp = pick_dvt(units, p->dk + p->dv, pl.f32);

  if (p->varlen)
    GDR_LAUNCH(GDR_KERNEL_PLAN, s, gdr::launch_plan(cu_seqlens, pl.N, p->seqlen, pl.NCb, (int*)(ws + pl.seq_chunk), (int*)(ws + pl.chunk_seq), s));
  if (pl.NCb > 0) {
    gdr::WyArgs wa{};
    wa.geo = geo; wa.DV = p->dv; wa.scale = scale;
    wa.q = q; wa.k = k; wa.v = v; wa.dO = dO; wa.beta = beta; wa.g = g;
    wa.gam = (float*)(ws + pl.gam);
    wa.gaml = (float*)(ws + pl.gaml);
    // W (fragment order) and U only feed the snapshot recompute
    wa.Wf = h_saved ? nullptr : (void*)(ws + pl.Wf);
    wa.Ua = h_saved ? nullptr : (float*)(ws + pl.Ua);
    wa.KtTf = h_saved ? nullptr : (void*)(ws + pl.KtTf);
    wa.Tm = (float*)(ws + pl.Tm); wa.WTf = ws + pl.WTf; wa.Kf = ws + pl.Kf;
    wa.dDl = (float*)(ws + pl.dDl); wa.Z = (float*)(ws + pl.Z);
    GDR_LAUNCH(GDR_KERNEL_WY, s, gdr::launch_wy(wa, pl.f32, p->dk, true, s));
    if (!h_saved) {
      gdr::ScanFwdArgs sa{};
      sa.geo = geo; sa.DV = p->dv; sa.layout = p->layout; sa.scale = scale; sa.h0 = h0; sa.hT = nullptr;
      sa.gam = (const float*)(ws + pl.gam); sa.Wf = ws + pl.Wf; sa.KtTf = ws + pl.KtTf; sa.Ua = (const float*)(ws + pl.Ua);
      sa.o = nullptr; sa.hs = ws + pl.hs;
      if (p->cp_segments > 1) {
        sa.summ = (float*)(ws + pl.summ); sa.hstart = (const float*)(ws + pl.hst);
        GDR_LAUNCH(GDR_KERNEL_CP_SCAN_FWD, s, gdr::launch_scan_fwd(sa, pl.f32, p->h_store_dtype, p->dk, dvt_cp, 0, s));
        gdr::CpChainArgs ca{geo, p->dk, p->dv, p->layout, 0, h0, (const float*)(ws + pl.summ), (float*)(ws + pl.hst)};
        GDR_LAUNCH(GDR_KERNEL_CP_CHAIN_FWD, s, gdr::launch_cp_chain(ca, s));
      }
      GDR_LAUNCH(GDR_KERNEL_SCAN_FWD, s, gdr::launch_scan_fwd(sa, pl.f32, p->h_store_dtype, p->dk, dvt, 1, s));
    }
  }
  gdr::ScanBwdArgs ba{};
  ba.geo = geo; ba.DV = p->dv; ba.layout = p->layout; ba.dhT = dhT; ba.dh0 = dh0;
  ba.gam = (const float*)(ws + pl.gam); ba.Kf = ws + pl.Kf; ba.WTf = ws + pl.WTf;
  ba.dDl = (const float*)(ws + pl.dDl); ba.Z = (const float*)(ws + pl.Z); ba.dhs = ws + pl.dhs; ba.dD = ws + pl.dD;
  if (p->cp_segments > 1) {
    // the forward recompute above is done with the hand-off buffer: reuse it
    ba.summ = (float*)(ws + pl.summ); ba.dhend = (const float*)(ws + pl.hst);
    GDR_LAUNCH(GDR_KERNEL_CP_SCAN_BWD, s, gdr::launch_scan_bwd(ba, pl.f32, p->dk, dvt_cp, 0, s));
    gdr::CpChainArgs ca{geo, p->dk, p->dv, p->layout, 1, dhT, (const float*)(ws + pl.summ), (float*)(ws + pl.hst)};
    GDR_LAUNCH(GDR_KERNEL_CP_CHAIN_BWD, s, gdr::launch_cp_chain(ca, s));
  }
  GDR_LAUNCH(GDR_KERNEL_SCAN_BWD, s, gdr::launch_scan_bwd(ba, pl.f32, p->dk, dvt, 1, s));
  if (pl.NCb > 0) {
    gdr::GradArgs ga{};
    ga.geo = geo; ga.DV = p->dv; ga.scale = scale;
    ga.q = q; ga.k = k; ga.v = v; ga.dO = dO; ga.beta = beta;
    ga.gam = (const float*)(ws + pl.gam); ga.gaml = (const float*)(ws + pl.gaml); ga.WTf = ws + pl.WTf; ga.Tm = (const float*)(ws + pl.Tm);
    ga.hs = hs; ga.dhs = ws + pl.dhs; ga.dD = ws + pl.dD;
    ga.dq = dq; ga.dk = dk; ga.dv = dv; ga.dbeta = dbeta; ga.dg = dg;
    GDR_LAUNCH(GDR_KERNEL_GRAD, s, gdr::launch_grad(ga, pl.f32, p->h_store_dtype, p->dk, s));
  }
  return GDR_OK;
}

const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
  }
  return "GDR_ERR_UNKNOWN";
}

const char* gdr_last_error(void) { return g_err; }

gdr_status gdr_validate_cu_seqlens(const int32_t* cu_seqlens, int num_seqs, int total_tokens, int32_t* result,
                                   void* stream) {
  g_err[0] = 0;
  if (!cu_seqlens || !result) { set_err("cu_seqlens and result are required"); return GDR_ERR_INVALID_ARG; }
  if (num_seqs < 1 || num_seqs > GDR_MAX_SEQS) {
    set_err("num_seqs must be in [1, %d] (got %d)", GDR_MAX_SEQS, num_seqs);
    return GDR_ERR_INVALID_ARG;
  }
  if (total_tokens < 0) { set_err("total_tokens must be >= 0 (got %d)", total_tokens); return GDR_ERR_INVALID_ARG; }
  if (((uintptr_t)cu_seqlens & 3) || ((uintptr_t)result & 3)) {
    set_err("cu_seqlens and result must be 4-byte aligned");
    return GDR_ERR_INVALID_ARG;
  }
  const hipError_t e = gdr::launch_check_cu(cu_seqlens, num_seqs, total_tokens, result, (hipStream_t)stream);
  if (e != hipSuccess) { set_err("launch failed: %s", hipGetErrorString(e)); return GDR_ERR_HIP; }
  return GDR_OK;
}

gdr_status gdr_set_kernel_timers(void* const* events) {
  g_err[0] = 0;
  if (!events) {
    g_timed = false;
    return GDR_OK;
  }
  for (int i = 0; i < 2 * GDR_NUM_KERNELS; ++i) g_events[i] = (hipEvent_t)events[i];
  g_timed = true;
  return GDR_OK;
}

int gdr_version(void) { return 100; }

#ifdef GDR_DEBUG_DELAY
gdr_status gdr_debug_set_delay(int wave, int mod, int iters, int salt) {
  g_err[0] = 0;
  if (wave < -1 || wave > 7 || mod < 1 || iters < 0 || iters > 64) {
    set_err("delay settings out of range (wave %d, mod %d, iters %d)", wave, mod, iters);
    return GDR_ERR_INVALID_ARG;
  }
  const gdr::DelayCfg c{wave, mod, iters, salt};
  GDR_TRY(gdr::debug_set_delay_fwd(c));
  GDR_TRY(gdr::debug_set_delay_bwd(c));
  GDR_TRY(gdr::debug_set_delay_rmsnorm(c));
  return GDR_OK;
}
#endif

}  // extern "C"
