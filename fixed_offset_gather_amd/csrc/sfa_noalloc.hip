// sfa_bwd_noalloc: the backward of the shared-offset attention for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  It runs the kernels of
// sfa_bwd with its workspace placed in `scratch`, a file-scope device array
// of SFA_NOALLOC_SCRATCH_BYTES that every device the library runs on holds
// until the process ends.
//
// Host code never uses the array's name as a device address: on each device
// (the first call made with that device current) hipGetSymbolAddress yields
// the device's own copy, and that pointer is kept per device and handed to
// the kernels, as sfa_bwd hands them the caller's workspace.  Nothing in the
// workspace has to start at zero (the query pass writes every entry the key
// pass and the reduction read), so no call clears it.  Calls that overlap on
// one device share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sfa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SFA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sfa::fail(SFA_ERR_HIP, "sfa_bwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return sfa::fail(SFA_ERR_UNSUPPORTED, "sfa_bwd_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return sfa::fail(SFA_ERR_HIP, "sfa_bwd_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SFA_OK;
}

}  // namespace

extern "C" int sfa_bwd_noalloc(const sfa_attn* a, const void* q, const void* k, const void* v, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, float* dd, const int32_t* base,
                               double alpha, float* dtheta, void* stream) {
  sfa::clear_error();
  // Validation and the size check first, before any HIP call.
  sfa::Problem p;
  if (int rc = sfa::validate_problem(a, &p)) return rc;
  const size_t need = sfa::bwd_workspace_bytes(a);
  if (need > SFA_NOALLOC_SCRATCH_BYTES)
    return sfa::fail(SFA_ERR_CAPACITY,
                     "sfa_bwd_noalloc: this problem needs %zu bytes of workspace, more than the %llu bytes of "
                     "static scratch; use sfa_bwd with a caller workspace",
                     need, (unsigned long long)SFA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = device_scratch(&ws)) return rc;
  return sfa::bwd_impl(a, q, k, v, lse, dout, dq, dk, dv, dd, base, alpha, dtheta, ws, SFA_NOALLOC_SCRATCH_BYTES,
                       stream, "sfa_bwd_noalloc");
}
