// attn_varlen_full_vjp_noalloc: the forward + full VJP call without a
// caller-given workspace, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid
// allocation).  Its workspace is one file-scope device array, `scratch`, of
// ATTN_NOALLOC_SCRATCH_BYTES bytes; each GPU the library runs on holds its own
// copy of it from the library's first use on that GPU until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current and kept in `g_scratch`; only that
// address is ever handed to the kernels.
//
// Every call on one GPU shares that GPU's array, and the array keeps what the
// last call left in it.  The call needs nothing in it to start at zero: the
// planner rewrites the plan, the zero block and every table before the kernels
// that read them, and every stored dS image and FP32 partial is written by
// the dK/dV kernel before the dQ kernel reads it.  Calls that overlap on one
// GPU (other streams, other threads) race on the array and must be ordered by
// the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_varlen.h"
#include "entry.hpp"

namespace {

constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

void* g_scratch[MAX_DEVICES] = {nullptr};
std::mutex g_scratch_mu;

// Device address of the current GPU's copy of `scratch` (set up on the first
// call on each device).
attn_status scratch_ptr(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return rga::set_error(ATTN_HIP_ERROR, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return rga::set_error(ATTN_HIP_ERROR, "device %d outside 0..%d", dev, MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return rga::set_error(ATTN_HIP_ERROR, "hipGetSymbolAddress(scratch): %s",
                            hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_varlen_full_vjp_noalloc(
    const attn_problem* p, const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
    const attn_tensor* dout, const attn_tensor* out, const attn_tensor* dq,
    const attn_tensor* dk, const attn_tensor* dv, float* lse, attn_stream_t stream) {
  rga::clear_error();
  size_t need = 0;
  const attn_status st = rga::min_workspace(p, ATTN_ENTRY_FULL_VJP, &need);
  if (st != ATTN_OK) return st;
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return rga::set_error(ATTN_WORKSPACE_TOO_SMALL,
                          "the problem needs %zu bytes of workspace; the static scratch holds %zu",
                          need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const attn_status sp = scratch_ptr(&ws);
  if (sp != ATTN_OK) return sp;
  // the whole array is the workspace: what the minimum layout leaves free
  // holds stored dS images, as in attn_varlen_full_vjp with a workspace of
  // ATTN_NOALLOC_SCRATCH_BYTES bytes
  return rga::full_vjp_impl(p, q, k, v, dout, out, dq, dk, dv, lse, ws,
                            (size_t)ATTN_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream),
                            nullptr);
}
