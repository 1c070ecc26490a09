// An allocation-free SwiGLU layer, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops).  It runs the
// same kernels as uw_mlp_forward with the gate/up outputs and h kept in a
// fixed device array instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "runtime_internal.h"

// The workspace of every call on a device: one copy per device, held until
// the process ends.  The host name of this array is only a stand-in for the
// device symbol; its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[UW_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up once per device
// (with that device current) and kept.
uw_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return uw::set_error(UW_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return uw::set_error(UW_ERR_NO_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return uw::set_error(UW_ERR_HIP, "hipGetSymbolAddress of the static workspace failed");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return UW_OK;
}

}  // namespace

extern "C" uw_status uw_mlp_forward_noalloc(uw_handle gate, uw_handle up, uw_handle down, const int32_t* pipelines,
                                            const uint16_t* x_dev, float* y_dev, int64_t tokens) {
  if (!gate) return uw::set_error(UW_ERR_INVALID_ARG, "null gate handle");
  uw_info gi;
  uw_status st = uw_query(gate, &gi);
  if (st != UW_OK) return st;
  if (tokens >= 1 && uw_mlp_workspace_bytes(tokens, gi.rows) > UW_STATIC_WORKSPACE_BYTES)
    return uw::set_error(UW_ERR_SHAPE,
                         "tokens x intermediate size needs more than the static workspace "
                         "(UW_STATIC_WORKSPACE_BYTES); use uw_mlp_forward with a workspace");
  void* work = nullptr;
  if ((st = scratch_of_current_device(&work)) != UW_OK) return st;
  return uw::mlp_forward_impl(gate, up, down, pipelines, x_dev, y_dev, tokens, work, UW_STATIC_WORKSPACE_BYTES,
                              true);
}
