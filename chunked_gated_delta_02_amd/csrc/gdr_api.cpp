// gdr_api.cpp -- host side of libgdr: argument validation, workspace layout,
// launch planning.  Implements the C ABI declared in include/libgdr.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

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
  if (p->cp_segments != 1) { set_err("intra-card context parallelism (cp_segments > 1) is not available in this build"); return GDR_ERR_UNSUPPORTED; }
  const double tokens = (double)p->batch * p->seqlen;
  if (tokens * p->heads * (p->dv > p->dk ? p->dv : p->dk) > 4.0e12) { set_err("problem too large"); return GDR_ERR_UNSUPPORTED; }
  return GDR_OK;
}

struct Plan {
  int N = 0, NCb = 0, ncps = 0;
  bool f32 = false;
  size_t esz = 2, hsz = 4;
  size_t seq_chunk = 0, chunk_seq = 0, gam = 0, Wf = 0, KtTf = 0, Ua = 0, hs = 0, Qgf = 0, Pf = 0;
  size_t Tm = 0, WTf = 0, PsTf = 0, QgsTf = 0, Ktf = 0, dOf = 0, dhs = 0, dD = 0;
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
  pl.Wf = take(ch * 64 * DK * e);
  pl.Ua = take(ch * 64 * DV * e);
  if (need_hs) {
    pl.hs = take(ch * DV * DK * pl.hsz);
    pl.KtTf = take(ch * DK * 64 * e);
  }
  if (mode == 0) {
    if (!need_hs) pl.KtTf = take(ch * DK * 64 * e);
    pl.Qgf = take(ch * 64 * DK * e);
    pl.Pf = take(ch * 64 * 64 * e);
  } else {
    pl.Tm = take(ch * 64 * 64 * 4);
    pl.WTf = take(ch * DK * 64 * e);
    pl.PsTf = take(ch * 64 * 64 * e);
    pl.QgsTf = take(ch * DK * 64 * e);
    pl.Ktf = take(ch * 64 * DK * e);
    pl.dOf = take(ch * DV * 64 * e);
    pl.dhs = take(ch * DK * DV * e);
    pl.dD = take(ch * 64 * DV * e);
  }
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
  return g;
}

// DV tile of the serial scans: the largest of 64 / 32 / 16 that still gives
// at least two workgroups per compute unit (512), else 16.  The fp32 path
// always uses 16 (its operand fragments are 8x larger per k).
int pick_dvt(int units, int dv, bool f32) {
  if (f32) return 16;
  if ((long)units * (dv / 64) >= 512) return 64;
  if ((long)units * (dv / 32) >= 512) return 32;
  return 16;
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

extern "C" {

gdr_status gdr_check(const gdr_problem* p) {
  g_err[0] = 0;
  return check_problem(p);
}

size_t gdr_fwd_workspace_bytes(const gdr_problem* p) {
  if (check_problem(p) != GDR_OK) return 0;
  return make_plan(p, 0, true).total;
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
  g_err[0] = 0;
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  const bool tokens = (int64_t)p->batch * p->seqlen > 0;
  if (tokens && (!q || !k || !v || !beta || !g || !o)) { set_err("q, k, v, beta, g and o are required"); return GDR_ERR_INVALID_ARG; }
  if ((p->varlen != 0) != (cu_seqlens != nullptr)) { set_err("cu_seqlens must be given exactly when varlen is 1"); return GDR_ERR_INVALID_ARG; }
  const void* ptrs[] = {q, k, v, beta, g, o, h0, hT, h_saved, cu_seqlens};
  for (const void* ptr : ptrs)
    if (ptr && misaligned(ptr)) { set_err("all buffers must be 16-byte aligned"); return GDR_ERR_INVALID_ARG; }
  const Plan pl = make_plan(p, 0, h_saved == nullptr);
  if (!workspace || workspace_bytes < pl.total) {
    set_err("workspace of %zu bytes needed (got %zu)", pl.total, workspace ? workspace_bytes : (size_t)0);
    return GDR_ERR_WORKSPACE;
  }
  char* ws = align_ws(workspace);
  hipStream_t s = (hipStream_t)stream;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->dk);
  gdr::Geo geo = make_geo(p, pl, cu_seqlens, ws);
  void* hs = h_saved ? h_saved : (void*)(ws + pl.hs);

  if (p->varlen)
    GDR_LAUNCH(GDR_KERNEL_PLAN, s, gdr::launch_plan(cu_seqlens, pl.N, p->seqlen, pl.NCb, (int*)(ws + pl.seq_chunk), (int*)(ws + pl.chunk_seq), s));
  if (pl.NCb > 0) {
    gdr::WyArgs wa{};
    wa.geo = geo; wa.DV = p->dv; wa.scale = scale;
    wa.q = q; wa.k = k; wa.v = v; wa.beta = beta; wa.g = g;
    wa.gam = (float*)(ws + pl.gam); wa.Wf = ws + pl.Wf; wa.KtTf = ws + pl.KtTf; wa.Ua = ws + pl.Ua;
    wa.Qgf = ws + pl.Qgf; wa.Pf = ws + pl.Pf;
    GDR_LAUNCH(GDR_KERNEL_WY, s, gdr::launch_wy(wa, pl.f32, p->dk, false, s));
  }
  gdr::ScanFwdArgs sa{};
  sa.geo = geo; sa.DV = p->dv; sa.layout = p->layout; sa.scale = scale; sa.h0 = h0; sa.hT = hT;
  sa.gam = (const float*)(ws + pl.gam); sa.Wf = ws + pl.Wf; sa.KtTf = ws + pl.KtTf; sa.Ua = ws + pl.Ua;
  sa.Qgf = ws + pl.Qgf; sa.Pf = ws + pl.Pf; sa.o = o; sa.hs = hs;
  GDR_LAUNCH(GDR_KERNEL_SCAN_FWD, s, gdr::launch_scan_fwd(sa, pl.f32, p->h_store_dtype, p->dk, pick_dvt(pl.N * p->heads, p->dv, pl.f32), s));
  return GDR_OK;
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
  if (tokens && (!q || !k || !v || !beta || !g || !dO || !dq || !dk || !dv || !dbeta || !dg)) {
    set_err("q, k, v, beta, g, dO, dq, dk, dv, dbeta and dg are required");
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
  const int dvt = pick_dvt(pl.N * p->heads, p->dv, pl.f32);

  if (p->varlen)
    GDR_LAUNCH(GDR_KERNEL_PLAN, s, gdr::launch_plan(cu_seqlens, pl.N, p->seqlen, pl.NCb, (int*)(ws + pl.seq_chunk), (int*)(ws + pl.chunk_seq), s));
  if (pl.NCb > 0) {
    gdr::WyArgs wa{};
    wa.geo = geo; wa.DV = p->dv; wa.scale = scale;
    wa.q = q; wa.k = k; wa.v = v; wa.dO = dO; wa.beta = beta; wa.g = g;
    wa.gam = (float*)(ws + pl.gam); wa.Wf = ws + pl.Wf; wa.Ua = ws + pl.Ua;
    wa.KtTf = h_saved ? nullptr : (void*)(ws + pl.KtTf);
    wa.Tm = (float*)(ws + pl.Tm); wa.WTf = ws + pl.WTf; wa.PsTf = ws + pl.PsTf; wa.QgsTf = ws + pl.QgsTf;
    wa.Ktf = ws + pl.Ktf; wa.dOf = ws + pl.dOf;
    GDR_LAUNCH(GDR_KERNEL_WY, s, gdr::launch_wy(wa, pl.f32, p->dk, true, s));
    if (!h_saved) {
      gdr::ScanFwdArgs sa{};
      sa.geo = geo; sa.DV = p->dv; sa.layout = p->layout; sa.scale = scale; sa.h0 = h0; sa.hT = nullptr;
      sa.gam = (const float*)(ws + pl.gam); sa.Wf = ws + pl.Wf; sa.KtTf = ws + pl.KtTf; sa.Ua = ws + pl.Ua;
      sa.Qgf = nullptr; sa.Pf = nullptr; sa.o = nullptr; sa.hs = ws + pl.hs;
      GDR_LAUNCH(GDR_KERNEL_SCAN_FWD, s, gdr::launch_scan_fwd(sa, pl.f32, p->h_store_dtype, p->dk, dvt, s));
    }
  }
  gdr::ScanBwdArgs ba{};
  ba.geo = geo; ba.DV = p->dv; ba.layout = p->layout; ba.dhT = dhT; ba.dh0 = dh0;
  ba.gam = (const float*)(ws + pl.gam); ba.Ktf = ws + pl.Ktf; ba.PsTf = ws + pl.PsTf; ba.QgsTf = ws + pl.QgsTf;
  ba.WTf = ws + pl.WTf; ba.dOf = ws + pl.dOf; ba.dhs = ws + pl.dhs; ba.dD = ws + pl.dD;
  GDR_LAUNCH(GDR_KERNEL_SCAN_BWD, s, gdr::launch_scan_bwd(ba, pl.f32, p->dk, dvt, s));
  if (pl.NCb > 0) {
    gdr::GradArgs ga{};
    ga.geo = geo; ga.DV = p->dv; ga.scale = scale;
    ga.q = q; ga.k = k; ga.v = v; ga.dO = dO; ga.beta = beta;
    ga.gam = (const float*)(ws + pl.gam); ga.Wf = ws + pl.Wf; ga.Ua = ws + pl.Ua; ga.Tm = (const float*)(ws + pl.Tm);
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

}  // extern "C"
