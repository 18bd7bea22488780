// moe_forward_noalloc: moe_forward with its workspace in a static device
// array instead of a caller-provided buffer (declared in moe.h).
//
// The array, `scratch`, is a file-scope __device__ variable of this
// translation unit: every GPU the library runs on holds its own copy from the
// time the code object is loaded on that GPU until the process ends.  On the
// host the name `scratch` is only a stand-in for the symbol, not a device
// address, so the host code never passes it anywhere: on the first call on a
// device, with that device current, hipGetSymbolAddress gives the device
// address of that device's copy, which is cached per device and is what the
// kernels receive (as moe_forward's workspace pointer).
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "moe.h"

namespace {

constexpr size_t kScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device (guarded by g_mu)

// Device address of the current device's scratch array.
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::record_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return moe::record_hip_error(e);
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_shape* shape, const moe_weights* w, float* y,
                                   int32_t* topk_ids, float* topk_w, void* stream) {
  int rc = moe::check_forward_args(shape, w, y, topk_ids, topk_w);
  if (rc) return rc;
  if (shape->T == 0) return MOE_OK;
  size_t need = 0;
  rc = moe_workspace_size(shape, &need);
  if (rc) return rc;
  if (need > kScratchBytes) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc) return rc;
  // moe_forward writes every workspace byte its kernels read within the same
  // call, so the array needs no clearing between calls
  return moe_forward(shape, w, y, topk_ids, topk_w, ws, kScratchBytes, stream);
}
