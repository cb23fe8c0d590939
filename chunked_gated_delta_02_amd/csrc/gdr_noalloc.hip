// gdr_noalloc.hip -- the allocation-free forward entry point,
// gdr_chunk_fwd_noalloc: the same kernels as gdr_chunk_fwd, with the
// workspace taken from a fixed device array of this library instead of a
// caller-provided buffer, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops).
//
// The array `scratch` has one copy per GPU, created when the library's code
// object is loaded on that GPU and kept until the process ends.  In host code
// its name is only a stand-in for the symbol: the device address is looked
// up once per device with hipGetSymbolAddress (that device current) and kept
// in g_ptr; only that address is ever handed to kernels.
//
// No workspace buffer of the forward has to start at zero: every one is
// written by an earlier launch of the same call before it is read (the
// chunk table of packed batches, the chunk intermediates, the context-
// parallel summaries and hand-off states), so the array is never cleared.
// All calls on one GPU share its array: calls whose launches can overlap on
// that GPU (different streams without ordering between them) race.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "gdr_host.h"

namespace {

constexpr size_t kScratchBytes = GDR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` on each GPU, once looked up

// device address of this GPU's `scratch`: looked up on the first call on a
// device, with that device current (it is the current device of the call)
gdr_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  char msg[256];
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "hipGetDevice failed: %s", hipGetErrorString(e));
    gdr::set_error(msg);
    return GDR_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof(msg), "device %d is beyond the %d devices the static workspace serves", dev, kMaxDevices);
    gdr::set_error(msg);
    return GDR_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
               hipGetErrorString(e));
      gdr::set_error(msg);
      return GDR_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v,
                                 const float* beta, const float* g, const int32_t* cu_seqlens,
                                 const float* h0, void* o, float* hT, void* h_saved, void* stream) {
  gdr::set_error("");
  const gdr_status st = gdr_check(p);
  if (st != GDR_OK) return st;
  const size_t need = gdr::fwd_workspace_bytes(p);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "problem needs %zu bytes of workspace, beyond the %zu of the static workspace of "
             "gdr_chunk_fwd_noalloc (use gdr_chunk_fwd with a caller-owned workspace)",
             need, kScratchBytes);
    gdr::set_error(msg);
    return GDR_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  const gdr_status s2 = scratch_of_current_device(&ws);
  if (s2 != GDR_OK) return s2;
  return gdr::chunk_fwd_impl(p, q, k, v, beta, g, cu_seqlens, h0, o, hT, h_saved, ws, kScratchBytes, stream);
}

}  // extern "C"
