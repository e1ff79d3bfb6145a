// Internal entry points of the library shared between its translation units
// (api.cpp holds the C ABI and defines them; noalloc.hip, the call with a
// static scratch, uses them).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_varlen.h"

namespace rga {

// Records the detail text of a failure for attn_last_error(); returns st.
attn_status set_error(attn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Minimum workspace of `entry` (attn_entry) for problem p (checks p first).
attn_status min_workspace(const attn_problem* p, int entry, size_t* bytes);

// The forward + full VJP call on a caller-given workspace (events: NULL or
// ATTN_PHASES + 1 events recorded before each phase and after the last).
attn_status full_vjp_impl(const attn_problem* p, const attn_tensor* q, const attn_tensor* k,
                          const attn_tensor* v, const attn_tensor* dout, const attn_tensor* out,
                          const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t s,
                          const hipEvent_t* ev);

}  // namespace rga
