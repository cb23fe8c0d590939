// gdr_host.h -- host-side internals shared by the entry points of libgdr.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "libgdr.h"

namespace gdr {

// the text gdr_last_error() returns on this thread
void set_error(const char* msg);
// workspace bytes the forward needs (the problem must have passed gdr_check)
size_t fwd_workspace_bytes(const gdr_problem* p);
// the forward on the given workspace: validation, then every launch on stream
gdr_status chunk_fwd_impl(const gdr_problem* p, const void* q, const void* k, const void* v,
                          const float* beta, const float* g, const int32_t* cu_seqlens,
                          const float* h0, void* o, float* hT, void* h_saved, void* workspace,
                          size_t workspace_bytes, void* stream);

}  // namespace gdr
