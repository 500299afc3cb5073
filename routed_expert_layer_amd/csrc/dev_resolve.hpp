// The shared expert cache's policy for one decode layer-step, on the device
// (page "FreeToken-rtx-4090", section "How the MoE Memory Hierarchy Works": one
// LRU over layer-and-expert keys shared across layers and tokens; page
// "FreeToken-benchmark", section "Graph Compatibility": the routing-dependent
// decisions live in device memory). The working set of a layer-step is its
// experts with at least one routed token, as keys layer*E + e; the keys
// resident at entry are hits and are touched first, ascending; the others are
// misses, touched next, ascending, each taking the lowest free slot, else the
// slot of the least recently used entry. Every touch takes the next value of
// a 64-bit clock as its slot's last use. The working set must fit the cache
// (the caller checks S >= min(E, k*T)), so a layer-step is a single wave.
// Used by the resolve kernel and by the decode-size routing kernel.
#pragma once
#include "dev_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace devctl {

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

// One layer-step of the policy, run by one whole workgroup of kResolveThreads threads (thread t < E takes
// expert t). count_of(e) / offset_of(e): the layer-step's row count and exclusive offset of expert e.
template <typename CountOf, typename OffsetOf>
__device__ __forceinline__ void resolve_layer_step(const int t, const int E, const int layer, const DevCache& c,
                                                   CountOf count_of, OffsetOf offset_of) {
  __shared__ int cnt[kResolveThreads / 64];
  __shared__ int miss_e[kResolveThreads];
  __shared__ uint64_t best_v[kResolveThreads / 64];
  __shared__ int best_s[kResolveThreads / 64];
  const uint64_t clock0 = c.ctl[0], seq = c.ctl[3], tr0 = c.ctl[4];
  const bool active = t < E && count_of(t) > 0;
  const int key = layer * E + t;
  const int slot0 = active ? c.slot_of[key] : -1;
  const bool hit = active && slot0 >= 0, miss = active && slot0 < 0;
  int n_hit, n_miss;
  const int hr = flag_rank(hit, cnt, n_hit);
  const int mr = flag_rank(miss, cnt, n_miss);
  if (hit) {
    c.stamp[slot0] = clock0 + 1 + hr;
    c.work[hr] = make_int4(slot0, offset_of(t), count_of(t), t);
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
      c.work[n_hit + j] = make_int4(slot, offset_of(e), count_of(e), e);
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

}  // namespace devctl
}  // namespace moe
