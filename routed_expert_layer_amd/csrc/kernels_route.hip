// Routing kernels: gate logits, wave-level top-k with softmax weights, and
// the stable grouping of (token, slot) pairs by expert.
//
// Page "FreeToken-rtx-4090", section "How the MoE Memory Hierarchy Works":
// each token activates a few of a layer's routed experts. The gate itself is
// not defined on the pages; these kernels compute the linear gate
// l = x.Wr + b, the k largest logits (ties to the lower expert index) and
// softmax weights renormalised over the selected k.
#include "dev_common.hpp"
#include "dev_resolve.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kRouterTok = 16;   // tokens per router block
constexpr int kMaxEPerLane = 16; // E <= 1024

template <bool BF16>
__device__ __forceinline__ float ldv(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

// Partial logits over a slice of H: partial[z][t][e] = sum_{h in slice z} x[t,h] Wr[h,e].
// Block: 256 threads = 4 groups of 64 experts-lanes; each group owns 4 tokens.
template <bool BF16>
__global__ __launch_bounds__(256) void router_partial_kernel(const void* __restrict__ x, const void* __restrict__ Wr,
                                                             int T, int H, int E, int hchunk,
                                                             float* __restrict__ partial) {
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int t0 = blockIdx.y * kRouterTok + grp * 4;
  const int h0 = blockIdx.z * hchunk;
  const int h1 = min(H, h0 + hchunk);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (e < E) {
    const int nt = min(4, T - t0);
    for (int h = h0; h < h1; ++h) {
      const float w = ldv<BF16>(Wr, (size_t)h * E + e);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nt) acc[i] = fmaf(ldv<BF16>(x, (size_t)(t0 + i) * H + h), w, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (t0 + i < T) partial[((size_t)blockIdx.z * T + t0 + i) * E + e] = acc[i];
  }
}

// Max of a 64-bit key over the wave. Inside each row of 16 lanes the
// butterfly uses DPP (quad permutes, then row rotations by 4 and 8); the four
// row maxima are then read with v_readlane.
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v, int ctrl_id) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint32_t lo2, hi2;
  switch (ctrl_id) {
    case 0:
      lo2 = __builtin_amdgcn_update_dpp(0, (int)lo, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
      hi2 = __builtin_amdgcn_update_dpp(0, (int)hi, 0xB1, 0xF, 0xF, false);
      break;
    case 1:
      lo2 = __builtin_amdgcn_update_dpp(0, (int)lo, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
      hi2 = __builtin_amdgcn_update_dpp(0, (int)hi, 0x4E, 0xF, 0xF, false);
      break;
    case 2:
      lo2 = __builtin_amdgcn_update_dpp(0, (int)lo, 0x124, 0xF, 0xF, false);  // row_ror:4
      hi2 = __builtin_amdgcn_update_dpp(0, (int)hi, 0x124, 0xF, 0xF, false);
      break;
    default:
      lo2 = __builtin_amdgcn_update_dpp(0, (int)lo, 0x128, 0xF, 0xF, false);  // row_ror:8
      hi2 = __builtin_amdgcn_update_dpp(0, (int)hi, 0x128, 0xF, 0xF, false);
      break;
  }
  uint64_t o = ((uint64_t)hi2 << 32) | lo2;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step(v, 0);
  v = dpp_max_step(v, 1);
  v = dpp_max_step(v, 2);
  v = dpp_max_step(v, 3);
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    best = o > best ? o : best;
  }
  return best;
}

// Order-preserving map of an fp32 value to uint32 (-0 is folded into +0 first).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// One wave per token: sum the partial logits, add the bias, select the top k
// by k rounds of a wave-wide maximum of (value, ~expert) keys, then the
// softmax weights over the selected logits.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int nsplit,
                                                   const float* __restrict__ bias, int T, int E, int k,
                                                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                   float* __restrict__ logits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // uniform per wave
  uint64_t key[kMaxEPerLane];
#pragma unroll
  for (int v = 0; v < kMaxEPerLane; ++v) {
    const int e = v * 64 + lane;
    key[v] = 0;
    if (e < E) {
      float l = 0.f;
      for (int z = 0; z < nsplit; ++z) l += partial[((size_t)z * T + t) * E + e];
      if (bias) l += bias[e];
      if (logits) logits[(size_t)t * E + e] = l;
      key[v] = ((uint64_t)float_key(l) << 32) | (uint32_t)(~(uint32_t)e);
    }
  }
  // k rounds; round j's winner is kept by lane j. The softmax denominator
  // is accumulated in round order from the (wave-uniform) winning values.
  float v0 = 0.f, den = 0.f, my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t local = 0;
#pragma unroll
    for (int v = 0; v < kMaxEPerLane; ++v) local = key[v] > local ? key[v] : local;
    const uint64_t best = wave_max_u64(local);
#pragma unroll
    for (int v = 0; v < kMaxEPerLane; ++v)
      if (key[v] == best) key[v] = 0;
    const float val = key_float((uint32_t)(best >> 32));
    if (j == 0) v0 = val;
    den += expf(val - v0);
    if (lane == j) {
      my_e = (int)(~(uint32_t)best);
      my_v = val;
    }
  }
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = expf(my_v - v0) / den;
  }
}

// Grouping of the T*k selections by expert, stable by token (three kernels
// over 64-token chunks, every step parallel over chunks or experts).
// Workspace: bits [nchunks][E] (which tokens of a chunk chose e), hist
// [E][nchunks] (their count, then the exclusive prefix over chunks).

// Exclusive prefix sum over a 256-thread block; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan256(int v, int* total) {
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(x, d);
    if (lane >= d) x += n;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(256) void chunk_masks_kernel(const int32_t* __restrict__ topk_idx, int T, int E, int k,
                                                          int nchunks, uint64_t* __restrict__ bits,
                                                          int32_t* __restrict__ hist) {
  extern __shared__ uint64_t bm[];  // E masks
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) bm[e] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * k; i += 256) {
    const int tl = i / k, j = i - tl * k, t = c * 64 + tl;
    if (t < T) atomicOr((unsigned long long*)&bm[topk_idx[(size_t)t * k + j]], 1ull << tl);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const uint64_t b = bm[e];
    bits[(size_t)c * E + e] = b;
    hist[(size_t)e * nchunks + c] = __popcll(b);
  }
}

// One block per expert: its chunk counts become exclusive prefixes, the
// total is the expert's count.
__global__ __launch_bounds__(256) void expert_scan_kernel(int32_t* __restrict__ hist, int nchunks,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ counts_mirror) {
  int32_t* h = hist + (size_t)blockIdx.x * nchunks;
  int carry = 0;
  for (int base = 0; base < nchunks; base += 256) {
    const int c = base + threadIdx.x;
    const int v = c < nchunks ? h[c] : 0;
    int tot;
    const int ex = block_excl_scan256(v, &tot);
    if (c < nchunks) h[c] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    counts[blockIdx.x] = carry;
    if (counts_mirror) counts_mirror[blockIdx.x] = carry;
  }
}

// One block per chunk: expert offsets (exclusive scan of the counts, redone
// by every block), then each selection's row = offset of its expert + rows
// of the expert in earlier chunks + earlier tokens of this chunk.
__global__ __launch_bounds__(256) void positions_kernel(const int32_t* __restrict__ topk_idx, int T, int E, int k,
                                                        int nchunks, const int32_t* __restrict__ counts,
                                                        const uint64_t* __restrict__ bits,
                                                        const int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                                                        int32_t* __restrict__ perm_pos) {
  extern __shared__ int32_t off[];  // E
  const int per = (E + 255) / 256;  // experts per thread, contiguous
  const int e0 = threadIdx.x * per;
  int local = 0;
  for (int q = 0; q < per; ++q)
    if (e0 + q < E) local += counts[e0 + q];
  int tot;
  int run = block_excl_scan256(local, &tot);
  for (int q = 0; q < per; ++q)
    if (e0 + q < E) {
      off[e0 + q] = run;
      if (blockIdx.x == 0) offsets[e0 + q] = run;
      run += counts[e0 + q];
    }
  if (blockIdx.x == 0 && threadIdx.x == 0) offsets[E] = tot;
  __syncthreads();
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < 64 * k; i += 256) {
    const int tl = i / k, j = i - tl * k, t = c * 64 + tl;
    if (t >= T) continue;
    const int e = topk_idx[(size_t)t * k + j];
    const uint64_t below = tl == 0 ? 0ull : (~0ull >> (64 - tl));
    const int pos = off[e] + hist[(size_t)e * nchunks + c] + __popcll(bits[(size_t)c * E + e] & below);
    perm_pos[(size_t)t * k + j] = pos;
    perm_src[pos] = t;
  }
}

// ---------------------------------------------------------------------------
// Decode-size batches (T <= 16, E <= 512): two launches in total.
// ---------------------------------------------------------------------------
constexpr int kSmallT = 16;
constexpr int kSmallE = 512;
constexpr int kSmallChunk = 64;  // rows of Wr per block

// partial[z][t][e] = sum over the block's 64 rows of x[t,h] Wr[h,e]. Wave w
// takes rows w, w+4, ..., w+60 of the block; lane l takes experts 4l..4l+3
// (+256 per pass), so each row is read as one coalesced 8-byte-per-lane
// access (bf16) and all 16 of a lane's row loads are in flight together. The
// four waves' sums are added in LDS in wave order.
template <bool BF16>
__global__ __launch_bounds__(256) void router_small_partial(const void* __restrict__ x, const void* __restrict__ Wr,
                                                            int T, int H, int E, float* __restrict__ partial) {
  __shared__ float xs[kSmallT][kSmallChunk];
  __shared__ float red[4][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h0 = blockIdx.x * kSmallChunk;
  const int nh = min(kSmallChunk, H - h0);
  auto load_w = [&](int e0, float (&w)[16][4]) {
    const int e = e0 + 4 * lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = wave + 4 * i;
#pragma unroll
      for (int c = 0; c < 4; ++c) w[i][c] = 0.f;
      if (h < nh) {
        const size_t base = (size_t)(h0 + h) * E + e;
        if (e + 3 < E && (E & 3) == 0) {
          if constexpr (BF16) {
            const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(Wr) + base);
            w[i][0] = __uint_as_float(v.x << 16);
            w[i][1] = __uint_as_float(v.x & 0xFFFF0000u);
            w[i][2] = __uint_as_float(v.y << 16);
            w[i][3] = __uint_as_float(v.y & 0xFFFF0000u);
          } else {
            const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(Wr) + base);
            w[i][0] = v.x;
            w[i][1] = v.y;
            w[i][2] = v.z;
            w[i][3] = v.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (e + c < E) w[i][c] = ldv<BF16>(Wr, base + c);
        }
      }
    }
  };
  // The first slab's weight loads go out before the activation barrier, so
  // both global reads overlap.
  float w[16][4];
  load_w(0, w);
  for (int i = threadIdx.x; i < T * kSmallChunk; i += 256) {
    const int t = i / kSmallChunk, h = i - t * kSmallChunk;
    xs[t][h] = h < nh ? ldv<BF16>(x, (size_t)t * H + h0 + h) : 0.f;
  }
  __syncthreads();
  const int tb = 1024 / (4 * 64);  // tokens per LDS reduction pass for one 256-expert slab: 4
  for (int e0 = 0; e0 < E; e0 += 256) {
    if (e0 > 0) load_w(e0, w);
    for (int t0 = 0; t0 < T; t0 += tb) {
      float acc[4][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[tt][c] = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = wave + 4 * i;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (t0 + tt < T && h < kSmallChunk) {
            const float xv = xs[t0 + tt][h];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[tt][c] = fmaf(xv, w[i][c], acc[tt][c]);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[wave][(tt * 64 + lane) * 4 + c] = acc[tt][c];
      __syncthreads();
      // 256 threads: thread -> (token tt, expert column) of this slab
      for (int q = threadIdx.x; q < 4 * 256; q += 256) {
        const int tt = q >> 8, col = q & 255;
        const int t = t0 + tt, ee = e0 + col;
        if (t < T && ee < E) {
          const int idx = (tt * 64 + (col >> 2)) * 4 + (col & 3);
          const float sum = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
          partial[((size_t)blockIdx.x * T + t) * E + ee] = sum;
        }
      }
      __syncthreads();
    }
  }
}

// Sum of p[z * stride] for z in [z0, z1), 16 independent accumulators added
// in a fixed order at the end.
__device__ __forceinline__ float sum_partials(const float* __restrict__ p, size_t stride, int z0, int z1) {
  float a[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) a[u] = 0.f;
  int z = z0;
  for (; z + 16 <= z1; z += 16) {
#pragma unroll
    for (int u = 0; u < 16; ++u) a[u] += p[(size_t)(z + u) * stride];
  }
  for (int u = 0; z < z1; ++z, ++u) a[u] += p[(size_t)z * stride];
#pragma unroll
  for (int u = 1; u < 16; ++u) a[0] += a[u];
  return a[0];
}

// One block: logits = sum of the partials + bias (fixed order), top-k of
// every token by one wave each, then the grouping of the <= 16 tokens.
__global__ __launch_bounds__(1024) void route_finish_small(const float* __restrict__ partial, int nsplit,
                                                           const float* __restrict__ bias, int T, int E, int k,
                                                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                           float* __restrict__ logits, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm_src,
                                                           int32_t* __restrict__ perm_pos,
                                                           int32_t* __restrict__ counts_mirror, int32_t mirror_seq,
                                                           const ResidentList res, const DevStep dev) {
  __shared__ float lg[kSmallT * kSmallE];
  __shared__ int32_t sidx[kSmallT * 16];
  __shared__ unsigned long long bm[kSmallE];
  __shared__ int32_t wsum[16];
  __shared__ int32_t soff[kSmallE];
  __shared__ float zsum[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float bias_first = (bias && tid < T * E) ? bias[tid % E] : 0.f;  // issued early
  for (int e = tid; e < E; e += 1024) bm[e] = 0ull;
  // the slot table copy's pending updates, for the kernels that follow (this kernel reads them from its
  // arguments, below)
  if (res.slot_of != nullptr && tid < res.updates.n) res.slot_of[res.updates.key[tid]] = res.updates.slot[tid];
  // logits: G threads per (t, e) each add a contiguous range of the partials
  // (16 loads in flight), then the G range sums are added in range order.
  {
    const int n = T * E;
    const int G = n <= 256 ? 4 : (n <= 512 ? 2 : 1);
    const int zper = (nsplit + G - 1) / G;
    if (G > 1) {
      if (tid < n * G) {
        const int i = tid % n, g = tid / n;
        zsum[tid] = sum_partials(partial + i, (size_t)n, g * zper, min(nsplit, (g + 1) * zper));
      }
      __syncthreads();
      if (tid < n) {
        float l = 0.f;
        for (int g = 0; g < G; ++g) l += zsum[g * n + tid];
        l += bias_first;
        lg[tid] = l;
        if (logits) logits[tid] = l;
      }
    } else {
      for (int i = tid; i < n; i += 1024) {
        float l = sum_partials(partial + i, (size_t)n, 0, nsplit);
        if (bias) l += i == tid ? bias_first : bias[i % E];
        lg[i] = l;
        if (logits) logits[i] = l;
      }
    }
  }
  __syncthreads();
  if (wave < T) {
    const int t = wave;
    uint64_t key[kSmallE / 64];
#pragma unroll
    for (int v = 0; v < kSmallE / 64; ++v) {
      const int e = v * 64 + lane;
      key[v] = e < E ? (((uint64_t)float_key(lg[t * E + e]) << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
    }
    float v0 = 0.f, den = 0.f, my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t local = 0;
#pragma unroll
      for (int v = 0; v < kSmallE / 64; ++v) local = key[v] > local ? key[v] : local;
      const uint64_t best = wave_max_u64(local);
#pragma unroll
      for (int v = 0; v < kSmallE / 64; ++v)
        if (key[v] == best) key[v] = 0;
      const float val = key_float((uint32_t)(best >> 32));
      if (j == 0) v0 = val;
      den += expf(val - v0);
      if (lane == j) {
        my_e = (int)(~(uint32_t)best);
        my_v = val;
      }
    }
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = expf(my_v - v0) / den;
      sidx[t * k + lane] = my_e;
      atomicOr(&bm[my_e], 1ull << t);
    }
  }
  __syncthreads();
  // counts and their exclusive prefix over experts (block scan)
  const int c = tid < E ? __popcll(bm[tid]) : 0;
  int v = c;
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(v, d);
    if (lane >= d) v += n;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int excl = before + v - c;
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = excl;
    soff[tid] = excl;
    // the host-mapped copy carries this launch's number in its upper half, so
    // each word shows by itself that it is current (no fence or flag needed)
    if (counts_mirror) counts_mirror[tid] = (int32_t)(((uint32_t)mirror_seq << 16) | (uint32_t)c);
  }
  if (tid == 0) offsets[E] = T * k;
  if (res.slot_of != nullptr) {
    // the experts with tokens that the slot table copy shows as resident, as FFN work items
    __shared__ int rcnt[16];
    int slot = -1;
    if (tid < E && c > 0) {
      const int key = res.layer * E + tid;
      slot = res.slot_of[key];
      for (int i = 0; i < res.updates.n; ++i)
        if (res.updates.key[i] == key) slot = res.updates.slot[i];
    }
    int total = 0, active = 0;
    const int r = block_flag_rank<16>(slot >= 0, rcnt, total);
    if (slot >= 0) res.items[r] = make_int4(slot, excl, c, tid);
    (void)block_flag_rank<16>(c > 0, rcnt, active);
    if (tid == 0) {
      res.n_out[0] = total;
      res.n_out[1] = active;
    }
  }
  __syncthreads();
  // positions: rank of a token inside its expert = earlier tokens in its mask
  if (tid < T * k) {
    const int t = tid / k, e = sidx[tid];
    const int pos = soff[e] + __popcll(bm[e] & ((1ull << t) - 1ull));
    perm_pos[tid] = pos;
    perm_src[pos] = t;
  }
  // a device-controlled decoder's resolve of this layer-step, from the counts and offsets in LDS
  if (dev.c.slot_of != nullptr)
    devctl::resolve_layer_step(
        tid, E, dev.layer, dev.c, [&](int e) { return __popcll(bm[e]); }, [&](int e) { return soff[e]; });
}

struct RoutePlan {
  int mode;  // 0: small (decode) path, 1: matrix-core path, 2: general VALU path
  int gx, gy, nsplit, hchunk;
  size_t partial_bytes, hist_off, bits_off, wrt_off, total;
};

bool gemm_router_ok(bool bf16, int T, int H, int E) {
  return bf16 && T > 64 && E % kGemmBN == 0 && H % 64 == 0;
}

RoutePlan plan_route(int T, int H, int E, bool bf16) {
  RoutePlan p{};
  const int nchunks = (T + 63) / 64;
  if (T <= kSmallT && E <= kSmallE) {
    p.mode = 0;
    p.nsplit = (H + kSmallChunk - 1) / kSmallChunk;
    p.partial_bytes = align_up((size_t)p.nsplit * (T > 0 ? T : 1) * E * sizeof(float), 256);
  } else if (gemm_router_ok(bf16, T, H, E)) {
    p.mode = 1;
    p.nsplit = router_gemm_splits(T, H, E);
    p.partial_bytes = align_up((size_t)p.nsplit * T * E * sizeof(float), 256);
  } else {
    p.mode = 2;
    p.gx = (E + 63) / 64;
    p.gy = (T + kRouterTok - 1) / kRouterTok;
    const int blocks = p.gx * (p.gy > 0 ? p.gy : 1);
    int ns = (512 + blocks - 1) / blocks;
    const int max_ns = H / 32 > 0 ? H / 32 : 1;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    p.hchunk = (H + ns - 1) / ns;
    p.nsplit = (H + p.hchunk - 1) / p.hchunk;
    p.partial_bytes = align_up((size_t)p.nsplit * T * E * sizeof(float), 256);
  }
  p.hist_off = p.partial_bytes;
  p.bits_off = align_up(p.hist_off + (size_t)nchunks * E * sizeof(int32_t), 256);
  p.wrt_off = align_up(p.bits_off + (size_t)nchunks * E * sizeof(uint64_t), 256);
  p.total = p.wrt_off + (p.mode == 1 ? align_up((size_t)H * E * 2, 256) : 0) + 256;
  return p;
}

}  // namespace

bool route_small_path(int T, int E) { return T <= kSmallT && E <= kSmallE; }

size_t route_workspace_bytes(int T, int H, int E, int k) {
  (void)k;
  // sized for the larger of the two element types
  const size_t a = plan_route(T, H, E, true).total, b = plan_route(T, H, E, false).total;
  return a > b ? a : b;
}

hipError_t launch_route(const void* x, bool bf16, const void* Wr, const float* bias, int T, int H, int E, int k,
                        int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts, int32_t* offsets,
                        int32_t* perm_src, int32_t* perm_pos, void* ws, hipStream_t s, int32_t* counts_mirror,
                        int32_t mirror_seq, const ResidentList* resident, const DevStep* dev) {
  const RoutePlan p = plan_route(T, H, E, bf16);
  ResidentList res{};
  if (resident != nullptr) {
    if (p.mode != 0 || resident->updates.n < 0 || resident->updates.n > kSlotUpdatesMax)
      return hipErrorInvalidValue;
    res = *resident;
  }
  DevStep dv{};
  if (dev != nullptr) {
    if (p.mode != 0 || E > devctl::kResolveThreads) return hipErrorInvalidValue;
    dv = *dev;
  }
  char* w = static_cast<char*>(ws);
  float* partial = reinterpret_cast<float*>(w);
  int32_t* hist = reinterpret_cast<int32_t*>(w + p.hist_off);
  uint64_t* bits = reinterpret_cast<uint64_t*>(w + p.bits_off);
  hipError_t err;
  if (p.mode == 0) {
    if (T > 0) {
      if (bf16)
        hipLaunchKernelGGL(router_small_partial<true>, dim3(p.nsplit), dim3(256), 0, s, x, Wr, T, H, E, partial);
      else
        hipLaunchKernelGGL(router_small_partial<false>, dim3(p.nsplit), dim3(256), 0, s, x, Wr, T, H, E, partial);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    hipLaunchKernelGGL(route_finish_small, dim3(1), dim3(1024), 0, s, partial, T > 0 ? p.nsplit : 0, bias, T, E, k,
                       topk_idx, topk_w, logits, counts, offsets, perm_src, perm_pos, counts_mirror, mirror_seq, res,
                       dv);
    return hipGetLastError();
  }
  if (p.mode == 1) {
    void* wrt = w + p.wrt_off;
    if ((err = launch_pack_fragments(Wr, H, E, wrt, s)) != hipSuccess) return err;
    if ((err = launch_router_gemm(x, wrt, T, H, E, partial, p.nsplit, s)) != hipSuccess) return err;
  } else {
    dim3 grid(p.gx, p.gy, p.nsplit);
    if (bf16)
      hipLaunchKernelGGL(router_partial_kernel<true>, grid, dim3(256), 0, s, x, Wr, T, H, E, p.hchunk, partial);
    else
      hipLaunchKernelGGL(router_partial_kernel<false>, grid, dim3(256), 0, s, x, Wr, T, H, E, p.hchunk, partial);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, partial, p.nsplit, bias,
                     T, E, k, topk_idx, topk_w, logits);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int nchunks = (T + 63) / 64;
  if (nchunks > 0) {
    hipLaunchKernelGGL(chunk_masks_kernel, dim3(nchunks), dim3(256), (size_t)E * 8, s, topk_idx, T, E, k, nchunks, bits,
                       hist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(expert_scan_kernel, dim3(E), dim3(256), 0, s, hist, nchunks, counts, counts_mirror);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(positions_kernel, dim3(nchunks > 0 ? nchunks : 1), dim3(256), (size_t)E * 4, s, topk_idx, T, E, k,
                     nchunks, counts, bits, hist, offsets, perm_src, perm_pos);
  return hipGetLastError();
}

}  // namespace moe
