// Device-resident control of the shared expert cache, so that a decode
// layer-step needs no host decision and can be replayed from a captured
// graph (page "FreeToken-benchmark", section "Graph Compatibility": the
// routing-dependent decisions live in device memory).
//
// The policy is the one the host cache applies (page "FreeToken-rtx-4090",
// section "How the MoE Memory Hierarchy Works": one LRU over layer-and-expert
// keys shared across layers and tokens): the working set of a layer-step is
// its experts with at least one routed token, as keys layer*E + e; the keys
// resident at entry are hits and are touched first, ascending; the others are
// misses, touched next, ascending, each taking the lowest free slot, else the
// slot of the least recently used entry. Every touch takes the next value of
// a 64-bit clock as its slot's last use. The working set must fit the cache
// (the caller checks S >= min(E, k*T)), so a layer-step is a single wave.
#include "dev_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kResolveThreads = 1024;
constexpr uint64_t kOccupied = 1ull << 62;  // slot order key: free slots (their index) before any stamp

__device__ __forceinline__ int flag_rank(bool f, int* cnt, int& total) {
  return block_flag_rank<kResolveThreads / 64>(f, cnt, total);
}

__device__ __forceinline__ void wave_argmin(uint64_t& v, int& s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t ov = __shfl_xor(v, off);
    const int os = __shfl_xor(s, off);
    if (ov < v || (ov == v && os < s)) {
      v = ov;
      s = os;
    }
  }
}

__device__ __forceinline__ void put_trace(const DevCache& c, uint64_t at, int32_t seq, int32_t layer, int32_t key,
                                          int32_t hit, int32_t slot, int32_t victim) {
  if (at >= (uint64_t)c.trace_cap) return;
  int32_t* r = c.trace + at * 7;
  r[0] = seq;
  r[1] = layer;
  r[2] = key;
  r[3] = hit;
  r[4] = slot;
  r[5] = victim;
  r[6] = 0;
}

// One workgroup. counts/offsets: the layer-step's per-expert row counts and
// exclusive offsets (device, from the routing kernels).
__global__ __launch_bounds__(kResolveThreads) void dev_resolve_kernel(const int32_t* __restrict__ counts,
                                                                      const int32_t* __restrict__ offsets, int E,
                                                                      int layer, DevCache c) {
  __shared__ int cnt[kResolveThreads / 64];
  __shared__ int miss_e[kResolveThreads];
  __shared__ uint64_t best_v[kResolveThreads / 64];
  __shared__ int best_s[kResolveThreads / 64];
  const int t = threadIdx.x;
  const uint64_t clock0 = c.ctl[0], seq = c.ctl[3], tr0 = c.ctl[4];
  const bool active = t < E && counts[t] > 0;
  const int key = layer * E + t;
  const int slot0 = active ? c.slot_of[key] : -1;
  const bool hit = active && slot0 >= 0, miss = active && slot0 < 0;
  int n_hit, n_miss;
  const int hr = flag_rank(hit, cnt, n_hit);
  const int mr = flag_rank(miss, cnt, n_miss);
  if (hit) {
    c.stamp[slot0] = clock0 + 1 + hr;
    c.work[hr] = make_int4(slot0, offsets[t], counts[t], t);
    put_trace(c, tr0 + hr, (int32_t)seq, layer, key, 1, slot0, -1);
  }
  if (miss) miss_e[mr] = t;
  __syncthreads();  // hit stamps and the miss list are visible to the whole block
  for (int j = 0; j < n_miss; ++j) {
    // lowest free slot, else least recently used (unique stamps)
    uint64_t bv = ~0ull;
    int bs = 0x7fffffff;
    for (int s = t; s < c.S; s += kResolveThreads) {
      const int k = c.slot_key[s];
      const uint64_t v = k < 0 ? (uint64_t)s : kOccupied + c.stamp[s];
      if (v < bv) {
        bv = v;
        bs = s;
      }
    }
    wave_argmin(bv, bs);
    if ((t & 63) == 0) {
      best_v[t >> 6] = bv;
      best_s[t >> 6] = bs;
    }
    __syncthreads();
    if (t == 0) {
      uint64_t v = best_v[0];
      int slot = best_s[0];
      for (int w = 1; w < kResolveThreads / 64; ++w)
        if (best_v[w] < v || (best_v[w] == v && best_s[w] < slot)) {
          v = best_v[w];
          slot = best_s[w];
        }
      const int e = miss_e[j], mkey = layer * E + e;
      const int victim = c.slot_key[slot];
      if (victim >= 0) c.slot_of[victim] = -1;
      c.slot_key[slot] = mkey;
      c.slot_of[mkey] = slot;
      c.stamp[slot] = clock0 + 1 + n_hit + j;
      c.work[n_hit + j] = make_int4(slot, offsets[e], counts[e], e);
      c.miss[j] = make_int4(e, slot, victim, mkey);
      put_trace(c, tr0 + n_hit + j, (int32_t)seq, layer, mkey, 0, slot, victim);
    }
    __syncthreads();  // this miss's slot is taken before the next search
  }
  if (t == 0) {
    c.n[0] = n_hit + n_miss;
    c.n[1] = n_miss;
    c.n[2] = n_hit;
    c.ctl[0] = clock0 + n_hit + n_miss;
    c.ctl[1] += n_hit;
    c.ctl[2] += n_miss;
    c.ctl[3] = seq + 1;
    c.ctl[4] = tr0 + n_hit + n_miss;
  }
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
  if (E > kResolveThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dev_resolve_kernel, dim3(1), dim3(kResolveThreads), 0, s, counts, offsets, E, layer, c);
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
