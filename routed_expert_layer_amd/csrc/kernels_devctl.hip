// Device-resident control of the shared expert cache, so that a decode
// layer-step needs no host decision and can be replayed from a captured
// graph (page "FreeToken-benchmark", section "Graph Compatibility": the
// routing-dependent decisions live in device memory). The policy itself, the
// one the host cache applies, is resolve_layer_step (dev_resolve.hpp).
#include "dev_common.hpp"
#include "dev_resolve.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// One workgroup. counts/offsets: the layer-step's per-expert row counts and
// exclusive offsets (device, from the routing kernels).
__global__ __launch_bounds__(devctl::kResolveThreads) void dev_resolve_kernel(const int32_t* __restrict__ counts,
                                                                              const int32_t* __restrict__ offsets,
                                                                              int E, int layer, DevCache c) {
  devctl::resolve_layer_step(
      (int)threadIdx.x, E, layer, c, [&](int e) { return counts[e]; }, [&](int e) { return offsets[e]; });
}

// Copies the layer-step's missing blobs from the host pool into their slots.
// A fixed grid walks 64 KiB chunks (16 bytes per thread and load, 16 loads in
// flight per thread); with no misses every block returns at once.
constexpr int kFillBlocks = 512;
constexpr int kFillChunk = 256 * 16 * 16;
__global__ __launch_bounds__(256) void dev_fill_kernel(const int32_t* __restrict__ n, const int4* __restrict__ miss,
                                                       const char* __restrict__ pool, size_t blob_stride,
                                                       size_t blob_bytes, char* __restrict__ slot_base,
                                                       size_t slot_stride) {
  const int nm = n[1];
  if (nm == 0) return;
  const size_t per = (blob_bytes + kFillChunk - 1) / kFillChunk;
  const size_t total = per * (size_t)nm;
  for (size_t ch = blockIdx.x; ch < total; ch += gridDim.x) {
    const int j = (int)(ch / per);
    const size_t off0 = (ch - (size_t)j * per) * kFillChunk;
    const int4 m = miss[j];
    const char* src = pool + (size_t)m.x * blob_stride + off0;
    char* dst = slot_base + (size_t)m.y * slot_stride + off0;
    const size_t lim = blob_bytes - off0;  // bytes of this blob from the chunk start
    u32x4_t v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const size_t o = ((size_t)q * 256 + threadIdx.x) * 16;
      if (o < lim) v[q] = ld16(src + o);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const size_t o = ((size_t)q * 256 + threadIdx.x) * 16;
      if (o < lim) *reinterpret_cast<u32x4_t*>(dst + o) = v[q];
    }
  }
}

// slot_of[key] = slot for each of the u.n distinct keys listed.
__global__ __launch_bounds__(64) void slot_update_kernel(int32_t* __restrict__ slot_of, const SlotUpdates u) {
  const int i = threadIdx.x;
  if (i < u.n) slot_of[u.key[i]] = u.slot[i];
}

}  // namespace

hipError_t launch_slot_updates(int32_t* slot_of, const SlotUpdates& u, hipStream_t s) {
  if (u.n <= 0) return hipSuccess;
  if (u.n > kSlotUpdatesMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(slot_update_kernel, dim3(1), dim3(64), 0, s, slot_of, u);
  return hipGetLastError();
}

hipError_t launch_dev_resolve(const int32_t* counts, const int32_t* offsets, int E, int layer, const DevCache& c,
                              hipStream_t s) {
  if (E > devctl::kResolveThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dev_resolve_kernel, dim3(1), dim3(devctl::kResolveThreads), 0, s, counts, offsets, E, layer, c);
  return hipGetLastError();
}

hipError_t launch_dev_fill(const DevCache& c, const void* pool, size_t blob_stride, size_t blob_bytes,
                           void* slot_base, size_t slot_stride, hipStream_t s) {
  if (blob_bytes % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dev_fill_kernel, dim3(kFillBlocks), dim3(256), 0, s, c.n, c.miss,
                     static_cast<const char*>(pool), blob_stride, blob_bytes, static_cast<char*>(slot_base),
                     slot_stride);
  return hipGetLastError();
}

}  // namespace moe
