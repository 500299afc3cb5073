// moe_route_noalloc: moe_route for callers that cannot allocate (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc). The
// routing kernels' scratch lives in one file-scope device array per GPU; the
// host finds its address on each device once and never uses the array's name
// as an address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_kernels.hpp"

namespace {

// Each GPU the library runs on holds this array until the process ends. No
// routing kernel needs it cleared (every byte it reads was written earlier in
// the same call).
constexpr size_t kScratchBytes = (size_t)MOE_ROUTE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on its first call there).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::set_error(MOE_EHIP, "moe_route_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return moe::set_error(MOE_EINVAL, "moe_route_noalloc: device %d not supported", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return moe::set_error(MOE_EHIP, "moe_route_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_route_noalloc(const void* x, int dtype, const void* Wr, const float* bias, int T, int H, int E,
                                 int k, int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts,
                                 int32_t* offsets, int32_t* perm_src, int32_t* perm_pos, void* stream) {
  const size_t need = moe_route_workspace_size(T, H, E, k);
  if (need > kScratchBytes)
    return moe::set_error(MOE_ECAPACITY,
                          "moe_route_noalloc: T=%d H=%d E=%d k=%d needs %zu bytes of scratch, more than the %zu the "
                          "library holds per GPU; use moe_route with a workspace",
                          T, H, E, k, need, kScratchBytes);
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != MOE_OK) return rc;
  return moe_route(x, dtype, Wr, bias, T, H, E, k, topk_idx, topk_w, logits, counts, offsets, perm_src, perm_pos, ws,
                   kScratchBytes, stream);
}
