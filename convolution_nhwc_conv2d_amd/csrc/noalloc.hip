// The allocation-free 2D forward entry point: cnhwc_conv2d_fwd with its
// workspace taken from a fixed device array that the library holds, for
// callers that cannot allocate device memory themselves (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives in this module's device data, one copy per GPU, from the
// module's load until the process ends.  Its host-side name only stands in for
// the symbol: the address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (that device current) and kept; only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cnhwc.h"

namespace cnhwc {
namespace {

static __device__ __align__(256) unsigned char scratch[CNHWC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Address of the current device's copy of the array (nullptr on a HIP error).
void* scratch_address(int dev) {
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace cnhwc

extern "C" cnhwc_status_t cnhwc_conv2d_fwd_noalloc(const cnhwc_conv_desc_t* desc,
                                                   const cnhwc_plan_t* plan, const void* x,
                                                   const void* w, void* y, void* hip_stream) {
  if (!desc || !plan) return CNHWC_ERR_INVALID_ARGUMENT;
  if (plan->workspace_bytes > CNHWC_NOALLOC_SCRATCH_BYTES) return CNHWC_ERR_WORKSPACE_TOO_SMALL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CNHWC_ERR_HIP;
  if (dev < 0 || dev >= cnhwc::kMaxDevices) return CNHWC_ERR_UNSUPPORTED;
  if (hip_stream) {
    // the array's address is per device: the stream must run on the current one
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev) != hipSuccess)
      return CNHWC_ERR_HIP;
    if (sdev != dev) return CNHWC_ERR_INVALID_ARGUMENT;
  }
  void* ws = nullptr;
  if (plan->workspace_bytes > 0) {
    ws = cnhwc::scratch_address(dev);
    if (!ws) return CNHWC_ERR_HIP;
  }
  return cnhwc_conv2d_fwd(desc, plan, x, w, y, ws, ws ? CNHWC_NOALLOC_SCRATCH_BYTES : 0,
                          hip_stream);
}
