// Grouped SwiGLU expert FFN: y = (silu(x W1) * (x W3)) W2 for each listed
// expert over its group of rows.
//
// Decode (few rows per expert) is bound by streaming the expert's weights
// from HBM: the matrix-vector kernels give each workgroup one 16-row tile of
// a weight matrix, split its K range over four waves, and feed every 1 KiB
// weight fragment straight from a coalesced global load into a 16x16x32
// matrix-core instruction whose other operand holds the (<= 16) tokens. A
// one-token bf16 step's down projection can instead run one workgroup per 16
// output columns over all of the step's experts, which lets it also form the
// step's weighted output (ffn2_combine_bf16).
// Prefill (many rows per expert) runs a tiled matrix-core GEMM with both
// operands staged in LDS.
#include <cstring>

#include "dev_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// Where a decode launch finds its work items {slot, row_begin, rows, expert}:
// in the kernel arguments (lists resolved on the host; the grid matches the
// list), or in device memory (lists resolved on the device; the grid is sized
// for the longest possible list and blocks past the list's length exit).
// src() gives the address item i's blob is read from and sets `fill` to an
// address the kernel also writes every byte it reads to (nullptr: none).
struct ArgWork {
  static constexpr bool kMayFill = false;
  WorkArgs wa;
  __device__ __forceinline__ bool get(int i, int4& it) const {
    it = wa.item[i];
    return true;
  }
  __device__ __forceinline__ const char* src(int, const int4& it, const char* slot_base, size_t slot_stride,
                                             char*& fill) const {
    fill = nullptr;
    return slot_base + (size_t)it.x * slot_stride;
  }
};
// A work list in device memory: *n items; the grid is sized for the most there can be and surplus blocks exit.
struct DevList {
  const int32_t* n;
  const int4* items;
  __device__ __forceinline__ bool get(int i, int4& it) const {
    if (i >= *n) return false;
    const int4 v = items[i];  // the same item for the whole block: keep it in scalar registers
    it = make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                   __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
    return true;
  }
};
// Resident experts only: every item's blob is in its slot, so the kernels built for this source have no
// write-through path (fewer registers, so more waves per SIMD, and half the LDS of the DevWork ones).
struct DevHits : DevList {
  static constexpr bool kMayFill = false;
  __device__ __forceinline__ const char* src(int, const int4& it, const char* slot_base, size_t slot_stride,
                                             char*& fill) const {
    fill = nullptr;
    return slot_base + (size_t)it.x * slot_stride;
  }
  // src with the number of hits read once by the caller (hits())
  __device__ __forceinline__ int hits() const { return kFuseItems; }
  __device__ __forceinline__ const char* src_at(int i, int, const int4& it, const char* slot_base,
                                                size_t slot_stride, char*& fill) const {
    return src(i, it, slot_base, slot_stride, fill);
  }
};
// With `pool` set, items from *n_hit on are misses: their blob is read from the
// host pool (pool + expert * pool_stride, device-visible pinned memory) and
// written through into their slot, so the fill and the FFN are one pass.
struct DevWork : DevList {
  static constexpr bool kMayFill = true;
  const int32_t* n_hit;
  const char* pool;
  size_t pool_stride;
  __device__ __forceinline__ const char* src(int i, const int4& it, const char* slot_base, size_t slot_stride,
                                             char*& fill) const {
    char* slot = const_cast<char*>(slot_base) + (size_t)it.x * slot_stride;
    if (pool != nullptr && i >= *n_hit) {
      fill = slot;
      return pool + (size_t)it.w * pool_stride;
    }
    fill = nullptr;
    return slot;
  }
  // src with the number of hits read once by the caller (hits())
  __device__ __forceinline__ int hits() const { return pool != nullptr ? *n_hit : kFuseItems; }
  __device__ __forceinline__ const char* src_at(int i, int nh, const int4& it, const char* slot_base,
                                                size_t slot_stride, char*& fill) const {
    char* slot = const_cast<char*>(slot_base) + (size_t)it.x * slot_stride;
    if (pool != nullptr && i >= nh) {
      fill = slot;
      return pool + (size_t)it.w * pool_stride;
    }
    fill = nullptr;
    return slot;
  }
};

__device__ __forceinline__ void st16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Write-through of a miss (its blob read over the host link and stored into its slot as the FFN uses it):
// after the stores, wait until every memory operation of the wave has completed, before any loaded register
// is used. The compiler's wait counts take the wave's loads and stores to complete in issue order; with loads
// from host memory and stores to HBM, registers were read before their loads had returned (seen as NaN
// outputs of the int4 miss path), and a full wait does not depend on that order.
__device__ __forceinline__ void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }

// The result of a chain of matrix-core products moved to vector registers (which waits for the chain), with no
// instruction scheduled across that point.
__device__ __forceinline__ void matrix_chain_done(f32x4_t& v) {
  asm volatile("" : "+v"(v));
  __builtin_amdgcn_sched_barrier(0);
}

// A pointer every lane of the wave holds (a work item's blob) moved to scalar registers, as a buffer resource
// needs.
__device__ __forceinline__ char* uniform(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<char*>(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// fp32 weights: plain VALU kernels (small correctness configurations).
// ---------------------------------------------------------------------------
template <typename W>
__global__ __launch_bounds__(256) void ffn1_f32_kernel(const float* __restrict__ x, const int32_t* __restrict__ perm_src,
                                                       const W wk, const char* __restrict__ slot_base,
                                                       size_t slot_stride, int H, int I, float* __restrict__ hbuf) {
  int4 it;
  if (!wk.get(blockIdx.y, it)) return;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int m = idx / I, i = idx - (idx / I) * I;
  if (m >= it.z) return;
  const float* W1 = reinterpret_cast<const float*>(slot_base + (size_t)it.x * slot_stride);
  const float* W3 = W1 + (size_t)H * I;
  const float* xr = x + (size_t)perm_src[it.y + m] * H;
  float g = 0.f, u = 0.f;
  for (int h = 0; h < H; ++h) {
    g = fmaf(xr[h], W1[(size_t)h * I + i], g);
    u = fmaf(xr[h], W3[(size_t)h * I + i], u);
  }
  hbuf[(size_t)(it.y + m) * I + i] = silu(g) * u;
}

template <typename W>
__global__ __launch_bounds__(256) void ffn2_f32_kernel(const float* __restrict__ hbuf, const W wk,
                                                       const char* __restrict__ slot_base, size_t slot_stride, int H,
                                                       int I, float* __restrict__ y) {
  int4 it;
  if (!wk.get(blockIdx.y, it)) return;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int m = idx / H, n = idx - (idx / H) * H;
  if (m >= it.z) return;
  const float* W2 = reinterpret_cast<const float*>(slot_base + (size_t)it.x * slot_stride) + 2 * (size_t)H * I;
  const float* hr = hbuf + (size_t)(it.y + m) * I;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(hr[i], W2[(size_t)i * H + n], acc);
  y[(size_t)(it.y + m) * H + n] = acc;
}

// ---------------------------------------------------------------------------
// bf16 decode kernels.
// ---------------------------------------------------------------------------
constexpr int kU = 8;  // fragments in flight per wave

// How a decode kernel reads its 16-byte activation fragments: plain loads, or loads coherent across the
// device's XCDs (for SwiGLU products another block of the same launch has just written through).
struct PlainLoad {
  __device__ __forceinline__ u32x4_t operator()(const uint16_t* p) const { return ld16(p); }
};
struct CoherentLoad {
  const uint16_t* base;  // wave-uniform; every address read lies within 2^32 bytes above it
  __device__ __forceinline__ u32x4_t operator()(const uint16_t* p) const {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, -1, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)((const char*)p - (const char*)base), 0,
                                                 16);  // sc1: device scope
  }
};


// One wave's share of a tile: the sum over fragments [c0, c1) (1 KiB apart
// from wp) of each fragment times the activation fragment at ar + 32c. With
// WT every weight fragment is also stored at the same offset from fp (the
// write-through of a miss); the stores follow each batch's loads, and the
// variant without them keeps its loads free to move.
template <bool WT, typename ALoad = PlainLoad>
__device__ __forceinline__ f32x4_t bf16_wave_dot(const char* wp, char* fp, const uint16_t* ar, bool valid, int c0,
                                                 int c1, ALoad aload = ALoad()) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int c = c0;
  for (; c + kU <= c1; c += kU) {
    u32x4_t a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      a[u] = ld16_nt(wp + (size_t)(c + u) * 1024);
      b[u] = valid ? aload(ar + (c + u) * 32) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (WT) {
#pragma unroll
      for (int u = 0; u < kU; ++u) st16(fp + (size_t)(c + u) * 1024, a[u]);
      drain_memory();
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc = mfma_bf16(a[u], b[u], acc);
  }
  // The n < kU remaining fragments also go out as one batch: slots past the
  // end load the last fragment again (a cache hit) against a zero activation.
  const int n = c1 - c;
  if (n > 0) {
    u32x4_t a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int cu = c + (u < n ? u : n - 1);
      a[u] = ld16_nt(wp + (size_t)cu * 1024);
      b[u] = (valid && u < n) ? aload(ar + cu * 32) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (WT) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (u < n) st16(fp + (size_t)(c + u) * 1024, a[u]);
      drain_memory();
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc = mfma_bf16(a[u], b[u], acc);
  }
  return acc;
}

// Gate/up: workgroup = one 16-row tile of P1 (8 gate + 8 up columns) of one
// item; wave w reduces fragments [KC*w/4, KC*(w+1)/4). Each row's pair of
// SwiGLU products (two bf16 in one word) goes to store(address, word).
template <typename W, typename Store, typename ALoad = PlainLoad>
__device__ __forceinline__ void bf16_ffn1_tile(const uint16_t* x, const int32_t* perm_src, const W& wk, int item,
                                               const int4& it, int tile, const char* slot_base, size_t slot_stride,
                                               int H, int I, uint16_t* hbuf, Store store, ALoad aload = ALoad()) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KC = H / 32;
  const int c0 = (KC * wave) >> 2, c1 = (KC * (wave + 1)) >> 2;
  char* fill;
  const size_t toff = (size_t)tile * KC * 1024 + lane * 16;
  const char* wp = wk.src(item, it, slot_base, slot_stride, fill) + toff;
  char* fp = fill ? fill + toff : nullptr;
  const int kq = (lane >> 4) * 8;
  __shared__ f32x4_t red[4][64];
  for (int m0 = 0; m0 < it.z; m0 += 16) {
    const int m = m0 + (lane & 15);
    const bool valid = m < it.z;
    const uint16_t* xr = x + (size_t)(valid ? perm_src[it.y + m] : 0) * H + kq;
    const f32x4_t acc = fp ? bf16_wave_dot<true>(wp, fp, xr, valid, c0, c1, aload)
                           : bf16_wave_dot<false>(wp, nullptr, xr, valid, c0, c1, aload);
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && valid) {
      const f32x4_t s = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
      const int i0 = 8 * tile + 2 * (lane >> 4);
      const uint32_t packed =
          (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16);
      store(reinterpret_cast<uint32_t*>(hbuf + (size_t)(it.y + m) * I + i0), packed);
    }
    __syncthreads();
  }
}

// Down projection: workgroup = one 16-row tile of P2 (16 output columns).
template <typename W, typename ALoad = PlainLoad>
__device__ __forceinline__ void bf16_ffn2_tile(const uint16_t* hbuf, const W& wk, int item, const int4& it, int tile,
                                               const char* slot_base, size_t slot_stride, size_t p2_off, int H,
                                               int I, float* y, ALoad aload = ALoad()) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KC = I / 32;
  const int c0 = (KC * wave) >> 2, c1 = (KC * (wave + 1)) >> 2;
  char* fill;
  const size_t toff = p2_off + (size_t)tile * KC * 1024 + lane * 16;
  const char* wp = wk.src(item, it, slot_base, slot_stride, fill) + toff;
  char* fp = fill ? fill + toff : nullptr;
  const int kq = (lane >> 4) * 8;
  __shared__ f32x4_t red[4][64];
  for (int m0 = 0; m0 < it.z; m0 += 16) {
    const int m = m0 + (lane & 15);
    const bool valid = m < it.z;
    const uint16_t* hr = hbuf + (size_t)(it.y + (valid ? m : 0)) * I + kq;
    const f32x4_t acc = fp ? bf16_wave_dot<true>(wp, fp, hr, valid, c0, c1, aload)
                           : bf16_wave_dot<false>(wp, nullptr, hr, valid, c0, c1, aload);
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && valid) {
      const f32x4_t s = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
      *reinterpret_cast<f32x4_t*>(y + (size_t)(it.y + m) * H + 16 * tile + 4 * (lane >> 4)) = s;
    }
    __syncthreads();
  }
}

template <typename W>
__global__ __launch_bounds__(256) void ffn1_decode_bf16(const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ perm_src, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride, int H,
                                                        int I, uint16_t* __restrict__ hbuf) {
  const int NT = I / 8;
  const int item = blockIdx.x / NT, tile = blockIdx.x - item * NT;
  int4 it;
  if (!wk.get(item, it)) return;
  bf16_ffn1_tile(x, perm_src, wk, item, it, tile, slot_base, slot_stride, H, I, hbuf,
                 [](uint32_t* p, uint32_t v) { *p = v; });
}

template <typename W>
__global__ __launch_bounds__(256) void ffn2_decode_bf16(const uint16_t* __restrict__ hbuf, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride,
                                                        size_t p2_off, int H, int I, float* __restrict__ y) {
  const int NT = H / 16;
  const int item = blockIdx.x / NT, tile = blockIdx.x - item * NT;
  int4 it;
  if (!wk.get(item, it)) return;
  bf16_ffn2_tile(hbuf, wk, item, it, tile, slot_base, slot_stride, p2_off, H, I, y);
}

// Down projection and weighted combine of up to kFuseItems resident experts,
// in one launch: workgroup = 16 output columns (one 16-row tile of every
// item's P2), sixteen waves each taking F = I / 512 consecutive fragments of
// every item, two items per batch of loads. The waves' partial tiles meet in
// LDS and are summed in wave order; each item's rows go to y as in
// ffn2_decode_bf16 and to an LDS copy indexed by permuted row. When every
// expert of the step is listed (*n_active == *wk.n), the block then forms its
// 16 columns of out[t] = sum over j of w[t, j] y[pos[t, j]], j ascending, the
// combine kernel's own arithmetic, so the separate combine launch is not
// needed.
constexpr int kFuseWaves = 16, kFuseRows = 128;
template <typename W, int F>
__global__ __launch_bounds__(1024) void ffn2_combine_bf16(const uint16_t* __restrict__ hbuf, const W wk,
                                                          const char* __restrict__ slot_base, size_t slot_stride,
                                                          size_t p2_off, int H, int I, float* __restrict__ y,
                                                          const int32_t* __restrict__ n_active,
                                                          const int32_t* __restrict__ perm_pos,
                                                          const float* __restrict__ topk_w, int T, int k,
                                                          void* __restrict__ out, int out_bf16) {
  static_assert(F >= 1 && 2 * F <= kU, "two items' fragments per batch");
  __shared__ f32x4_t red[kFuseWaves][kFuseItems][64];
  __shared__ float ylds[kFuseRows][16];
  const int tile = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int KC = I / 32;
  // the list's size and its hits (later items are misses read from the pool), read once, so that no weight
  // load in the loop waits on them
  const int n = min(*wk.n, kFuseItems), nh = wk.hits();
  const int m = lane & 15, kq = (lane >> 4) * 8;
  const size_t toff = p2_off + ((size_t)tile * KC + (size_t)F * wave) * 1024 + lane * 16;
  for (int i = 0; i < n; i += 2) {
    const bool two = i + 1 < n;
    int4 ia, ib;
    (void)wk.get(i, ia);
    if (two) (void)wk.get(i + 1, ib);
    char *fa = nullptr, *fb = nullptr;
    const char* wa = wk.src_at(i, nh, ia, slot_base, slot_stride, fa) + toff;
    const bool va = m < ia.z;
    const uint16_t* ha = hbuf + (size_t)(ia.y + (va ? m : 0)) * I + kq + 32 * F * wave;
    u32x4_t a[2 * F], b[2 * F];
#pragma unroll
    for (int u = 0; u < F; ++u) {
      a[u] = ld16_nt(wa + (size_t)u * 1024);
      b[u] = va ? ld16(ha + 32 * u) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (two) {
      const char* wb = wk.src_at(i + 1, nh, ib, slot_base, slot_stride, fb) + toff;
      const bool vb = m < ib.z;
      const uint16_t* hb = hbuf + (size_t)(ib.y + (vb ? m : 0)) * I + kq + 32 * F * wave;
#pragma unroll
      for (int u = 0; u < F; ++u) {
        a[F + u] = ld16_nt(wb + (size_t)u * 1024);
        b[F + u] = vb ? ld16(hb + 32 * u) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    if (fa != nullptr || fb != nullptr) {  // a miss's fragments, read from the pool, go into its slot too
      if (fa != nullptr) {
#pragma unroll
        for (int u = 0; u < F; ++u) st16(fa + toff + (size_t)u * 1024, a[u]);
      }
      if (fb != nullptr) {
#pragma unroll
        for (int u = 0; u < F; ++u) st16(fb + toff + (size_t)u * 1024, a[F + u]);
      }
      drain_memory();
    }
    f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < F; ++u) sa = mfma_bf16(a[u], b[u], sa);
    if (two) {
#pragma unroll
      for (int u = 0; u < F; ++u) sb = mfma_bf16(a[F + u], b[F + u], sb);
    }
    red[wave][i][lane] = sa;
    if (two) red[wave][i + 1][lane] = sb;
  }
  __syncthreads();
  if (wave < n) {  // item `wave`: its 16 x 16 tile summed over the waves in order
    int4 it;
    (void)wk.get(wave, it);
    f32x4_t sum = red[0][wave][lane];
#pragma unroll
    for (int v = 1; v < kFuseWaves; ++v) sum += red[v][wave][lane];
    if (m < it.z) {
      const int row = it.y + m;
      *reinterpret_cast<f32x4_t*>(y + (size_t)row * H + 16 * tile + 4 * (lane >> 4)) = sum;
      *reinterpret_cast<f32x4_t*>(&ylds[row][4 * (lane >> 4)]) = sum;
    }
  }
  __syncthreads();
  if (*n_active != n) return;  // a missing expert's rows come later; the step's combine runs on its own
  const int tid = threadIdx.x;
  if (tid < T * 16) {
    const int t = tid >> 4, c = tid & 15;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(topk_w[t * k + j], ylds[perm_pos[t * k + j]][c], acc);
    const size_t o = (size_t)t * H + 16 * tile + c;
    if (out_bf16)
      reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(acc);
    else
      reinterpret_cast<float*>(out)[o] = acc;
  }
}

// ---------------------------------------------------------------------------
// int4 decode kernels (bf16 activations and SwiGLU product as in the bf16
// path; codes enter bf16 matrix-core products exactly as 1 + n/16, and each
// 128-row block's sum is formed as 16 t - 24 u in fp32 -- t the product with
// the biased codes, u the block's sum of the activations -- times that
// block's fp16 scale).
// ---------------------------------------------------------------------------

// The registers of one 128-wide K block: activation fragments, and the codes
// and the four rows' scales of each of the block's kRI tiles.
constexpr int kRI = 4;  // 16-row tiles per int4 block
struct Int4Stage {
  u32x4_t b[4];
  u32x4_t a[kRI];
  uint32_t sc0[kRI], sc1[kRI];
};

// Shared body of both int4 projections. A block owns kRI consecutive 16-row
// tiles of one expert; its four waves split K, and each wave applies every
// activation fragment it loads to all kRI tiles (one activation load per kRI
// KiB of codes). A wave keeps the next K block's loads in flight while it
// works on the current one. Partial sums meet in LDS; wave w finishes tiles w, w + 4, ...
// act_row(m): bf16 activations of row m of the group; the finished 16 x 16
// tile sums go to `emit(tile, m, sum)`. With WT every code and scale loaded
// is also stored at the same offset from qf_base / sf_base (the write-through
// of a miss), after each K block's loads.
template <bool WT, typename Row, typename Emit, typename ALoad = PlainLoad>
__device__ __forceinline__ void int4_decode_tiles(Row act_row, const int4 it, int K, const char* q_base,
                                                  const char* s_base, char* qf_base, char* sf_base, int tile0,
                                                  Emit emit, ALoad aload = ALoad()) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int KG = K / 128;
  const int g0 = (KG * wave) >> 2, g1 = (KG * (wave + 1)) >> 2;
  const int kq = (lane >> 4) * 8;
  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  // Codes and scales through buffer resources: one lane offset in a vector register, the (uniform) block
  // offsets in scalar registers, so a wave's loads of two K blocks cost few address registers.
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(uniform(q_base), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(uniform(s_base), (short)0, -1, 0x00020000);
  const int vq = lane * 16, vs = (lane >> 4) * 8;
  __shared__ f32x4_t red[4][kRI][64];
  for (int m0 = 0; m0 < it.z; m0 += 16) {
    const int m = m0 + (lane & 15);
    const bool valid = m < it.z;
    const uint16_t* ar = act_row(valid ? m : 0) + kq;
    f32x4_t acc[kRI];
#pragma unroll
    for (int r = 0; r < kRI; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Lanes past the group read the group's first row: a token's column of a product depends only on its own
    // activation column, and the columns of those lanes are never stored.
    auto load = [&](int g, Int4Stage& st) {
#pragma unroll
      for (int j = 0; j < 4; ++j) st.b[j] = aload(ar + 128 * g + 32 * j);
#pragma unroll
      for (int r = 0; r < kRI; ++r) {
        const int blk = (tile0 + r) * KG + g;
        st.a[r] = __builtin_amdgcn_raw_buffer_load_b128(rq, vq, blk * 1024, 2);  // non-temporal
        // The four fp16 scales are read as two 32-bit words and widened one by
        // one (a two-element fp16 vector view of the 64-bit load was
        // miscompiled into mixed-precision FMAs that all read the first word).
        const u32x2_t sc = __builtin_amdgcn_raw_buffer_load_b64(rs, vs, blk * 32, 0);
        st.sc0[r] = sc[0];
        st.sc1[r] = sc[1];
      }
      if constexpr (WT) {  // codes by every lane, each 8-byte scale group by one lane
        const __amdgpu_buffer_rsrc_t wq = __builtin_amdgcn_make_buffer_rsrc(uniform(qf_base), (short)0, -1,
                                                                            0x00020000);
        const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(uniform(sf_base), (short)0, -1,
                                                                            0x00020000);
#pragma unroll
        for (int r = 0; r < kRI; ++r) {
          const int blk = (tile0 + r) * KG + g;
          __builtin_amdgcn_raw_buffer_store_b128(st.a[r], wq, vq, blk * 1024, 0);
          if ((lane & 15) == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(st.sc0[r], ws, vs, blk * 32, 0);
            __builtin_amdgcn_raw_buffer_store_b32(st.sc1[r], ws, vs + 4, blk * 32, 0);
          }
        }
        drain_memory();
      }
    };
    // Each chain of four dependent products is read out before the next chain starts (matrix_chain_done), so
    // the first, independent product of a chain never waits in the matrix pipe behind the previous chain while
    // the conversions that follow it rewrite its A-operand registers: with the chains back to back, the first
    // tile's results came out wrong (seen on the miss path at K = 256, where a wave has one K block).
    auto compute = [&](const Int4Stage& st) {
      f32x4_t u = {0.f, 0.f, 0.f, 0.f};  // every row: the block's sum of this token's activations
#pragma unroll
      for (int j = 0; j < 4; ++j) u = mfma_bf16(ones, st.b[j], u);
      matrix_chain_done(u);
      const float u24 = -24.f * u[0];
#pragma unroll
      for (int r = 0; r < kRI; ++r) {
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) t = mfma_bf16(int4x8_to_bf16x8_biased(st.a[r][j]), st.b[j], t);
        matrix_chain_done(t);
        acc[r][0] = fmaf(fmaf(t[0], 16.f, u24), f16_bits_to_f32(st.sc0[r] & 0xFFFFu), acc[r][0]);
        acc[r][1] = fmaf(fmaf(t[1], 16.f, u24), f16_bits_to_f32(st.sc0[r] >> 16), acc[r][1]);
        acc[r][2] = fmaf(fmaf(t[2], 16.f, u24), f16_bits_to_f32(st.sc1[r] & 0xFFFFu), acc[r][2]);
        acc[r][3] = fmaf(fmaf(t[3], 16.f, u24), f16_bits_to_f32(st.sc1[r] >> 16), acc[r][3]);
      }
    };
    Int4Stage s0, s1;
    int g = g0;
    if (g < g1) load(g, s0);
    for (; g + 1 < g1; g += 2) {
      load(g + 1, s1);
      compute(s0);
      if (g + 2 < g1) load(g + 2, s0);
      compute(s1);
    }
    if (g < g1) compute(s0);
#pragma unroll
    for (int r = 0; r < kRI; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (valid) {
#pragma unroll
      for (int t = wave; t < kRI; t += 4) {
        const f32x4_t sum = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
        emit(tile0 + t, m, sum);
      }
    }
    __syncthreads();
  }
}

template <typename W>
__global__ __launch_bounds__(256) void ffn1_decode_int4(const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ perm_src, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride,
                                                        size_t p1s_off, int H, int I, uint16_t* __restrict__ hbuf) {
  const int NB = I / 8 / kRI;  // blocks per expert
  const int item = blockIdx.x / NB, tile0 = (blockIdx.x - item * NB) * kRI;
  int4 it;
  if (!wk.get(item, it)) return;
  char* fill;
  const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
  const int lane = threadIdx.x & 63;
  const auto row = [&](int m) { return x + (size_t)perm_src[it.y + m] * H; };
  const auto emit = [&](int tile, int m, const f32x4_t& s) {
    const int i0 = 8 * tile + 2 * (lane >> 4);
    const uint32_t packed =
        (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16);
    *reinterpret_cast<uint32_t*>(hbuf + (size_t)(it.y + m) * I + i0) = packed;
  };
  if (fill)
    int4_decode_tiles<true>(row, it, H, blob, blob + p1s_off, fill, fill + p1s_off, tile0, emit);
  else
    int4_decode_tiles<false>(row, it, H, blob, blob + p1s_off, nullptr, nullptr, tile0, emit);
}

template <typename W>
__global__ __launch_bounds__(256) void ffn2_decode_int4(const uint16_t* __restrict__ hbuf, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride,
                                                        size_t p2_off, size_t p2s_off, int H, int I,
                                                        float* __restrict__ y) {
  const int NB = H / 16 / kRI;
  const int item = blockIdx.x / NB, tile0 = (blockIdx.x - item * NB) * kRI;
  int4 it;
  if (!wk.get(item, it)) return;
  char* fill;
  const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
  const int lane = threadIdx.x & 63;
  const auto row = [&](int m) { return hbuf + (size_t)(it.y + m) * I; };
  const auto emit = [&](int tile, int m, const f32x4_t& s) {
    *reinterpret_cast<f32x4_t*>(y + (size_t)(it.y + m) * H + 16 * tile + 4 * (lane >> 4)) = s;
  };
  if (fill)
    int4_decode_tiles<true>(row, it, I, blob + p2_off, blob + p2s_off, fill + p2_off, fill + p2s_off, tile0, emit);
  else
    int4_decode_tiles<false>(row, it, I, blob + p2_off, blob + p2s_off, nullptr, nullptr, tile0, emit);
}

// ---------------------------------------------------------------------------
// MXFP4 decode kernels (bf16 activations; every FP4 code times its power-of-two
// block scale is exact in bf16, so the weights enter bf16 matrix-core
// instructions exactly and the result equals a bf16-weight product with the
// dequantised weights).
// ---------------------------------------------------------------------------

constexpr int kR = 4;  // 16-row tiles per MXFP4 block

// Eight FP4 codes (nibbles in K order) times 2^(e - 127) as the bf16 A operand.
__device__ __forceinline__ u32x4_t fp4x8_to_bf16x8(uint32_t w, float scale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

// E8M0 byte (1..254) to the fp32 power of two it encodes.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float((e & 0xFFu) << 23); }

// Shared body of both MXFP4 projections, organised as the int4 one: a block
// owns kR consecutive 16-row tiles of one expert, its four waves split the
// 128-wide K blocks, and each activation fragment loaded serves all kR tiles.
// act: bf16 activations; row m of the group is act_row(m). Finished 16 x 16
// tile sums go to `emit(tile, m, sum)`. With WT every code and scale loaded
// is also stored at the same offset from qf_base / sf_base (the write-through
// of a miss), after each K block's loads.
template <bool WT, bool PIPE = false, typename Row, typename Emit, typename ALoad = PlainLoad>
__device__ __forceinline__ void mxfp4_decode_tiles(Row act_row, const int4 it, int K, const char* q_base,
                                                   const char* s_base, char* qf_base, char* sf_base, int tile0,
                                                   Emit emit, ALoad aload = ALoad()) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KG = K / 128;
  const int g0 = (KG * wave) >> 2, g1 = (KG * (wave + 1)) >> 2;
  const int kq = (lane >> 4) * 8;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(uniform(q_base), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(uniform(s_base), (short)0, -1, 0x00020000);
  __shared__ f32x4_t red[4][kR][64];
  for (int m0 = 0; m0 < it.z; m0 += 16) {
    const int m = m0 + (lane & 15);
    const bool valid = m < it.z;
    const uint16_t* ar = act_row(valid ? m : 0) + kq;
    f32x4_t acc[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // one K block's activation fragments, codes and scales; with PIPE the next block's are loaded before the
    // current one is used (the one-launch FFN, whose down projection reads its activations past the L2)
    struct Stage {
      u32x4_t b[4];
      u32x4_t a[kR];
      uint32_t sc[kR];
    };
    // codes and scales through buffer resources (a lane offset in a vector register, the block offsets in
    // scalar registers), so two stages of loads cost few address registers
    auto load = [&](int g, Stage& st) {
#pragma unroll
      for (int j = 0; j < 4; ++j) st.b[j] = valid ? aload(ar + 128 * g + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int blk = (tile0 + r) * KG + g;
        st.a[r] = __builtin_amdgcn_raw_buffer_load_b128(rq, lane * 16, blk * 1024, 2);  // non-temporal
        st.sc[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, (lane & 15) * 4, blk * 64, 0);
      }
      if constexpr (WT) {  // codes by every lane, the scale block by lanes 0..15
        const __amdgpu_buffer_rsrc_t wq =
            __builtin_amdgcn_make_buffer_rsrc(uniform(qf_base), (short)0, -1, 0x00020000);
        const __amdgpu_buffer_rsrc_t ws =
            __builtin_amdgcn_make_buffer_rsrc(uniform(sf_base), (short)0, -1, 0x00020000);
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int blk = (tile0 + r) * KG + g;
          __builtin_amdgcn_raw_buffer_store_b128(st.a[r], wq, lane * 16, blk * 1024, 0);
          if (lane < 16) __builtin_amdgcn_raw_buffer_store_b32(st.sc[r], ws, lane * 4, blk * 64, 0);
        }
        drain_memory();
      }
    };
    auto compute = [&](const Stage& st) {
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[r] = mfma_bf16(fp4x8_to_bf16x8(st.a[r][j], e8m0_to_f32(st.sc[r] >> (8 * j))), st.b[j], acc[r]);
    };
    if constexpr (PIPE) {
      Stage s0, s1;
      int g = g0;
      if (g < g1) load(g, s0);
      for (; g + 1 < g1; g += 2) {
        load(g + 1, s1);
        compute(s0);
        if (g + 2 < g1) load(g + 2, s0);
        compute(s1);
      }
      if (g < g1) compute(s0);
    } else {  // one stage through plain loads (four waves per SIMD; faster here than buffer loads)
      for (int g = g0; g < g1; ++g) {
        u32x4_t b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = valid ? aload(ar + 128 * g + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
        u32x4_t a[kR];
        uint32_t sc[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const size_t blk = (size_t)(tile0 + r) * KG + g;
          a[r] = ld16_nt(q_base + blk * 1024 + lane * 16);
          sc[r] = *reinterpret_cast<const uint32_t*>(s_base + blk * 64 + (lane & 15) * 4);
        }
        if constexpr (WT) {  // codes by every lane, the scale block by lanes 0..15
#pragma unroll
          for (int r = 0; r < kR; ++r) {
            const size_t blk = (size_t)(tile0 + r) * KG + g;
            st16(qf_base + blk * 1024 + lane * 16, a[r]);
            if (lane < 16) *reinterpret_cast<uint32_t*>(sf_base + blk * 64 + lane * 4) = sc[r];
          }
          drain_memory();
        }
#pragma unroll
        for (int r = 0; r < kR; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[r] = mfma_bf16(fp4x8_to_bf16x8(a[r][j], e8m0_to_f32(sc[r] >> (8 * j))), b[j], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (valid) {
      const f32x4_t sum = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];
      emit(tile0 + wave, m, sum);
    }
    __syncthreads();
  }
}

template <typename W>
__global__ __launch_bounds__(256) void ffn1_decode_mxfp4(const uint16_t* __restrict__ x,
                                                         const int32_t* __restrict__ perm_src, const W wk,
                                                         const char* __restrict__ slot_base, size_t slot_stride,
                                                         size_t p1s_off, int H, int I, uint16_t* __restrict__ hbuf) {
  const int NB = I / 8 / kR;  // blocks per expert
  const int item = blockIdx.x / NB, tile0 = (blockIdx.x - item * NB) * kR;
  int4 it;
  if (!wk.get(item, it)) return;
  char* fill;
  const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
  const int lane = threadIdx.x & 63;
  const auto row = [&](int m) { return x + (size_t)perm_src[it.y + m] * H; };
  const auto emit = [&](int tile, int m, const f32x4_t& s) {
    const int i0 = 8 * tile + 2 * (lane >> 4);
    const uint32_t packed =
        (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16);
    *reinterpret_cast<uint32_t*>(hbuf + (size_t)(it.y + m) * I + i0) = packed;
  };
  if (fill)
    mxfp4_decode_tiles<true>(row, it, H, blob, blob + p1s_off, fill, fill + p1s_off, tile0, emit);
  else
    mxfp4_decode_tiles<false>(row, it, H, blob, blob + p1s_off, nullptr, nullptr, tile0, emit);
}

template <typename W>
__global__ __launch_bounds__(256) void ffn2_decode_mxfp4(const uint16_t* __restrict__ hbuf, const W wk,
                                                         const char* __restrict__ slot_base, size_t slot_stride,
                                                         size_t p2_off, size_t p2s_off, int H, int I,
                                                         float* __restrict__ y) {
  const int NB = H / 16 / kR;
  const int item = blockIdx.x / NB, tile0 = (blockIdx.x - item * NB) * kR;
  int4 it;
  if (!wk.get(item, it)) return;
  char* fill;
  const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
  const int lane = threadIdx.x & 63;
  const auto row = [&](int m) { return hbuf + (size_t)(it.y + m) * I; };
  const auto emit = [&](int tile, int m, const f32x4_t& s) {
    *reinterpret_cast<f32x4_t*>(y + (size_t)(it.y + m) * H + 16 * tile + 4 * (lane >> 4)) = s;
  };
  if (fill)
    mxfp4_decode_tiles<true>(row, it, I, blob + p2_off, blob + p2s_off, fill + p2_off, fill + p2s_off, tile0, emit);
  else
    mxfp4_decode_tiles<false>(row, it, I, blob + p2_off, blob + p2s_off, nullptr, nullptr, tile0, emit);
}

// Both projections of a decode step (bf16: WF 1, one tile per block; int4: WF
// 2 and MXFP4: WF 3, four) in one launch, for experts listed in device memory:
// blocks [0, G1) (G1 = max_items * NB1) run the gate/up tile groups as
// ffn1_decode_*, the others the down-projection groups as ffn2_decode_*. With
// a write-through work source, misses are read from the pool and stored into
// their slots as in those kernels. A gate/up block, once its SwiGLU products
// are stored, marks its group done for this call (flags[item * NB1 + group] =
// seq); a down-projection block waits until every group of its item carries
// seq and then reads the products. Products and flags are written and read
// with device-scope (sc1) accesses, so the hand-off holds whichever XCDs ran
// the blocks. A down-projection block waits only for blocks of lower index,
// and each XCD dispatches its share of the grid in index order, so every
// gate/up block it waits for has been dispatched, and gate/up blocks wait for
// nothing: every wait ends. The wait is still bounded (2^18 polls), after
// which the block goes on and its output is wrong rather than the GPU hung.
// The launch saves the second launch's start-up and lets down-projection
// blocks start while the gate/up tail drains.
constexpr int kQuantTiles = 4;  // tiles per block of both quantised kernels (kRI, kR)

// The gate/up part of one block (tile group `group` of item `item`) of ffn_decode_fused, its SwiGLU products
// stored with device-scope stores.
template <int WF, typename W>
__device__ __forceinline__ void fused_gate_up(const uint16_t* x, const int32_t* perm_src, const W& wk, int item,
                                              const int4& it, int group, const char* slot_base, size_t slot_stride,
                                              size_t p1s_off, int H, int I, uint16_t* hbuf) {
  const auto store = [](uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  if constexpr (WF == 1) {
    bf16_ffn1_tile(x, perm_src, wk, item, it, group, slot_base, slot_stride, H, I, hbuf, store);
  } else {
    const int lane = threadIdx.x & 63;
    char* fill;
    const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
    const auto row = [&](int m) { return x + (size_t)perm_src[it.y + m] * H; };
    const auto emit = [&](int tile, int m, const f32x4_t& s) {
      const int i0 = 8 * tile + 2 * (lane >> 4);
      store(reinterpret_cast<uint32_t*>(hbuf + (size_t)(it.y + m) * I + i0),
            (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16));
    };
    const int tile0 = group * kQuantTiles;
    if constexpr (WF == 2) {
      if (W::kMayFill && fill != nullptr)
        int4_decode_tiles<true>(row, it, H, blob, blob + p1s_off, fill, fill + p1s_off, tile0, emit);
      else
        int4_decode_tiles<false>(row, it, H, blob, blob + p1s_off, nullptr, nullptr, tile0, emit);
    } else {
      if (W::kMayFill && fill != nullptr)
        mxfp4_decode_tiles<true, true>(row, it, H, blob, blob + p1s_off, fill, fill + p1s_off, tile0, emit);
      else
        mxfp4_decode_tiles<false, true>(row, it, H, blob, blob + p1s_off, nullptr, nullptr, tile0, emit);
    }
  }
}

// The down-projection part of one block of ffn_decode_fused, the products read with device-scope loads.
template <int WF, typename W>
__device__ __forceinline__ void fused_down(const W& wk, int item, const int4& it, int group, const char* slot_base,
                                           size_t slot_stride, size_t p2_off, size_t p2s_off, int H, int I,
                                           const uint16_t* hbuf, float* y) {
  const CoherentLoad coh{hbuf};
  if constexpr (WF == 1) {
    bf16_ffn2_tile(hbuf, wk, item, it, group, slot_base, slot_stride, p2_off, H, I, y, coh);
  } else {
    const int lane = threadIdx.x & 63;
    char* fill;
    const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
    const auto row = [&](int m) { return hbuf + (size_t)(it.y + m) * I; };
    const auto emit = [&](int tile, int m, const f32x4_t& s) {
      *reinterpret_cast<f32x4_t*>(y + (size_t)(it.y + m) * H + 16 * tile + 4 * (lane >> 4)) = s;
    };
    const int tile0 = group * kQuantTiles;
    if constexpr (WF == 2) {
      if (W::kMayFill && fill != nullptr)
        int4_decode_tiles<true>(row, it, I, blob + p2_off, blob + p2s_off, fill + p2_off, fill + p2s_off, tile0,
                                emit, coh);
      else
        int4_decode_tiles<false>(row, it, I, blob + p2_off, blob + p2s_off, nullptr, nullptr, tile0, emit, coh);
    } else {
      if (W::kMayFill && fill != nullptr)
        mxfp4_decode_tiles<true, true>(row, it, I, blob + p2_off, blob + p2s_off, fill + p2_off, fill + p2s_off,
                                       tile0, emit, coh);
      else
        mxfp4_decode_tiles<false, true>(row, it, I, blob + p2_off, blob + p2s_off, nullptr, nullptr, tile0, emit,
                                        coh);
    }
  }
}

template <int WF, typename W>
__global__ __launch_bounds__(256) void ffn_decode_fused(const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ perm_src, const W wk,
                                                        int max_items, const char* __restrict__ slot_base,
                                                        size_t slot_stride, size_t p1s_off, size_t p2_off,
                                                        size_t p2s_off, int H, int I, uint16_t* hbuf,
                                                        float* __restrict__ y, uint64_t* flags, uint64_t seq_arg,
                                                        const uint64_t* seq_dev) {
  static_assert(kRI == kQuantTiles && kR == kQuantTiles, "one tile-group size for both 4-bit formats");
  // the call's flag value: given, or one above a counter in device memory that each call's earlier work
  // advances (never 0, the flags' initial value; 64 bits, so it does not wrap)
  const uint64_t seq = seq_dev != nullptr ? *seq_dev + 1u : seq_arg;
  constexpr int TPB = WF == 1 ? 1 : kQuantTiles;  // tiles per block
  const int NB1 = I / 8 / TPB, NB2 = H / 16 / TPB;
  const int G1 = max_items * NB1;
  int4 it;
  if ((int)blockIdx.x < G1) {
    const int item = blockIdx.x / NB1, group = blockIdx.x - item * NB1;
    if (!wk.get(item, it)) return;
    fused_gate_up<WF>(x, perm_src, wk, item, it, group, slot_base, slot_stride, p1s_off, H, I, hbuf);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's product stores have completed
    __syncthreads();                // ... and every wave's
    if (threadIdx.x == 0)
      __hip_atomic_store(flags + item * NB1 + group, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int b2 = blockIdx.x - G1, item = b2 / NB2, group = b2 - item * NB2;
  if (!wk.get(item, it)) return;
  if (threadIdx.x < 64) {  // one wave polls the item's gate/up groups
    const int lane = threadIdx.x;
    for (int spin = 0; spin < (1 << 18); ++spin) {
      bool done = true;
      for (int j = lane; j < NB1; j += 64)
        done &= __hip_atomic_load(flags + item * NB1 + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == seq;
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  fused_down<WF>(wk, item, it, group, slot_base, slot_stride, p2_off, p2s_off, H, I, hbuf, y);
}

// ---------------------------------------------------------------------------
// bf16 prefill GEMM. Tile: 128 weight rows x 128 tokens x 64 K, 4 waves each
// computing 64 x 64 with 16 matrix-core instructions per 32-wide K chunk.
// Both operands are staged in LDS in fragment order (two stages), so every
// LDS read is one conflict-free 16-byte access per lane.
// PHASE 1: A = gate/up rows (N = 2I, K = H), B = x rows through perm_src,
//          epilogue silu(gate) * up -> bf16 h.
// PHASE 2: A = down rows (N = H, K = I), B = h rows, epilogue -> fp32 y.
// PHASE 0: the router: A = Wr^T rows (N = E, K = H), B = x rows in order,
//          epilogue -> fp32 logits + bias.
// ---------------------------------------------------------------------------
template <int PHASE>
__global__ __launch_bounds__(256, 2) void ffn_gemm_bf16(const uint16_t* __restrict__ bsrc,
                                                       const int32_t* __restrict__ perm_src, const WorkArgs wa,
                                                       const char* __restrict__ slot_base, size_t slot_stride,
                                                       size_t mat_off, int N, int K, int H, int I,
                                                       uint16_t* __restrict__ hout, float* __restrict__ yout,
                                                       const float* __restrict__ bias) {
  __shared__ __attribute__((aligned(16))) char lds[2][32768];
  const int NTB = N / kGemmBN;
  const int mtg = blockIdx.x / NTB, nt = blockIdx.x - (blockIdx.x / NTB) * NTB;
  int item = 0;
  while (item + 1 < wa.n && wa.tile_prefix[item + 1] <= mtg) ++item;
  const int4 it = wa.item[item];
  const int mt = mtg - wa.tile_prefix[item];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wm = wave >> 1;
  const int KC = K / 32, KT = K / 64;
  const int ldb = (PHASE == 2) ? I : H;

  // A (weights): 16 fragments per stage, 4 per thread.
  const char* abase = slot_base + (size_t)it.x * slot_stride + mat_off;
  size_t a_off[4];
  int a_lds[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int id = r * 256 + tid, f = id >> 6, l = id & 63;
    a_off[r] = ((size_t)(nt * 8 + (f >> 1)) * KC + (f & 1)) * 1024 + l * 16;
    a_lds[r] = f * 1024 + l * 16;
  }
  // B (tokens): 128 rows x 64 K per stage, 4 x 16 bytes per thread.
  const uint16_t* brow[4];
  bool bval[4];
  int b_lds[4], b_k[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int id = r * 256 + tid, row = id >> 3, ch = id & 7;
    const int mloc = mt * kGemmBM + row;
    bval[r] = mloc < it.z;
    size_t src_row = 0;
    if (bval[r]) src_row = (PHASE == 1) ? (size_t)perm_src[it.y + mloc] : (size_t)(it.y + mloc);
    brow[r] = bsrc + src_row * ldb;
    b_k[r] = ch * 8;
    b_lds[r] = 16384 + ((row >> 4) * 2 + (ch >> 2)) * 1024 + ((ch & 3) * 16 + (row & 15)) * 16;
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) ra[r] = ld16(abase + a_off[r] + (size_t)kt * 2048);
#pragma unroll
    for (int r = 0; r < 4; ++r) rb[r] = bval[r] ? ld16(brow[r] + kt * 64 + b_k[r]) : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4_t*>(&lds[st][a_lds[r]]) = ra[r];
#pragma unroll
    for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4_t*>(&lds[st][b_lds[r]]) = rb[r];
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      u32x4_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4_t*>(&lds[st][((wn * 4 + i) * 2 + kc) * 1024 + lane * 16]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const u32x4_t*>(&lds[st][16384 + ((wm * 4 + j) * 2 + kc) * 1024 + lane * 16]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < KT) lstore(st ^ 1);
    __syncthreads();
  }

  // Epilogue.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int mloc = mt * kGemmBM + (wm * 4 + j) * 16 + (lane & 15);
    if (mloc >= it.z) continue;
    const size_t row = (size_t)(it.y + mloc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ntile = nt * 8 + wn * 4 + i;
      const f32x4_t s = acc[i][j];
      if constexpr (PHASE == 1) {
        const int i0 = 8 * ntile + 2 * (lane >> 4);
        const uint32_t packed =
            (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16);
        *reinterpret_cast<uint32_t*>(hout + row * I + i0) = packed;
      } else if constexpr (PHASE == 2) {
        *reinterpret_cast<f32x4_t*>(yout + row * H + 16 * ntile + 4 * (lane >> 4)) = s;
      } else {
        const int n0 = 16 * ntile + 4 * (lane >> 4);
        f32x4_t o = s;
        if (bias) {
          o[0] += bias[n0];
          o[1] += bias[n0 + 1];
          o[2] += bias[n0 + 2];
          o[3] += bias[n0 + 3];
        }
        *reinterpret_cast<f32x4_t*>(yout + row * N + n0) = o;
      }
    }
  }
}

}  // namespace

bool prefill_supported(int wfmt, int H, int I) {
  return wfmt == 1 && (2 * I) % kGemmBN == 0 && H % kGemmBN == 0 && H % 64 == 0 && I % 64 == 0;
}

namespace {

// The decode kernels of one format for `n_items` work items (the grid's item
// count) with at most `max_rows` rows each.
template <typename W>
hipError_t decode_kernels(int wfmt, const void* x, const int32_t* perm_src, const W& wk, int n_items, int max_rows,
                          const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                          hipStream_t s) {
  const BlobLayout L = blob_layout(wfmt, H, I);
  if (wfmt == 0) {
    if (max_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(ffn1_f32_kernel<W>, dim3((max_rows * I + 255) / 256, n_items), dim3(256), 0, s,
                       static_cast<const float*>(x), perm_src, wk, slot_base, slot_stride, H, I,
                       static_cast<float*>(hbuf));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ffn2_f32_kernel<W>, dim3((max_rows * H + 255) / 256, n_items), dim3(256), 0, s,
                       static_cast<const float*>(hbuf), wk, slot_base, slot_stride, H, I, y);
    return hipGetLastError();
  }
  if (wfmt == 1) {
    hipLaunchKernelGGL(ffn1_decode_bf16<W>, dim3(n_items * (I / 8)), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       perm_src, wk, slot_base, slot_stride, H, I, static_cast<uint16_t*>(hbuf));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ffn2_decode_bf16<W>, dim3(n_items * (H / 16)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(hbuf), wk, slot_base, slot_stride, L.p2, H, I, y);
    return hipGetLastError();
  }
  if (wfmt == 3) {
    hipLaunchKernelGGL(ffn1_decode_mxfp4<W>, dim3(n_items * (I / 8 / kR)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), perm_src, wk, slot_base, slot_stride, L.p1s, H, I,
                       static_cast<uint16_t*>(hbuf));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ffn2_decode_mxfp4<W>, dim3(n_items * (H / 16 / kR)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(hbuf), wk, slot_base, slot_stride, L.p2, L.p2s, H, I, y);
    return hipGetLastError();
  }
  // int4
  hipLaunchKernelGGL(ffn1_decode_int4<W>, dim3(n_items * (I / 8 / kRI)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), perm_src, wk, slot_base, slot_stride, L.p1s, H, I,
                     static_cast<uint16_t*>(hbuf));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ffn2_decode_int4<W>, dim3(n_items * (H / 16 / kRI)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(hbuf), wk, slot_base, slot_stride, L.p2, L.p2s, H, I, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_decode(int wfmt, const void* x, const int32_t* perm_src, const WorkArgs& wa,
                             const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                             hipStream_t s) {
  if (wa.n == 0) return hipSuccess;
  int max_rows = 0;
  for (int i = 0; i < wa.n; ++i) max_rows = wa.item[i].z > max_rows ? wa.item[i].z : max_rows;
  return decode_kernels(wfmt, x, perm_src, ArgWork{wa}, wa.n, max_rows, slot_base, slot_stride, H, I, hbuf, y, s);
}

hipError_t launch_ffn_decode_dev(int wfmt, const void* x, const int32_t* perm_src, const int32_t* n_items,
                                 const int4* items, int max_items, int max_rows, const char* slot_base,
                                 size_t slot_stride, int H, int I, void* hbuf, float* y, hipStream_t s,
                                 const int32_t* n_hit, const char* pool, size_t pool_stride) {
  if (max_items == 0) return hipSuccess;
  if (pool == nullptr)
    return decode_kernels(wfmt, x, perm_src, DevHits{{n_items, items}}, max_items, max_rows, slot_base, slot_stride,
                          H, I, hbuf, y, s);
  if (wfmt == 0) return hipErrorInvalidValue;  // the fp32 kernels do not write through
  return decode_kernels(wfmt, x, perm_src, DevWork{{n_items, items}, n_hit, pool, pool_stride}, max_items,
                        max_rows, slot_base, slot_stride, H, I, hbuf, y, s);
}

bool ffn_fused_ok(int wfmt, int H, int I) {
  if (wfmt == 1) return H % 32 == 0 && I % 32 == 0;
  return (wfmt == 2 || wfmt == 3) && H % (16 * kQuantTiles) == 0 && I % (8 * kQuantTiles) == 0;
}

size_t ffn_fused_flags(int max_items, int I) { return (size_t)max_items * (I / 8); }

namespace {

template <typename W>
hipError_t fused_kernel(int wfmt, const W& wk, const void* x, const int32_t* perm_src, int max_items,
                        const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y, uint64_t* flags,
                        uint64_t seq, const uint64_t* seq_dev, hipStream_t s) {
  const BlobLayout L = blob_layout(wfmt, H, I);
  const int tpb = wfmt == 1 ? 1 : kQuantTiles;
  const dim3 grid(max_items * (I / 8 / tpb + H / 16 / tpb));
  if (wfmt == 1)
    hipLaunchKernelGGL((ffn_decode_fused<1, W>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(x), perm_src, wk,
                       max_items, slot_base, slot_stride, L.p1s, L.p2, L.p2s, H, I, static_cast<uint16_t*>(hbuf), y,
                       flags, seq, seq_dev);
  else if (wfmt == 2)
    hipLaunchKernelGGL((ffn_decode_fused<2, W>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(x), perm_src, wk,
                       max_items, slot_base, slot_stride, L.p1s, L.p2, L.p2s, H, I, static_cast<uint16_t*>(hbuf), y,
                       flags, seq, seq_dev);
  else
    hipLaunchKernelGGL((ffn_decode_fused<3, W>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(x), perm_src, wk,
                       max_items, slot_base, slot_stride, L.p1s, L.p2, L.p2s, H, I, static_cast<uint16_t*>(hbuf), y,
                       flags, seq, seq_dev);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_decode_fused(int wfmt, const void* x, const int32_t* perm_src, const int32_t* n_items,
                                   const int4* items, int max_items, const char* slot_base, size_t slot_stride, int H,
                                   int I, void* hbuf, float* y, uint64_t* flags, uint64_t seq, hipStream_t s,
                                   const uint64_t* seq_dev, const int32_t* n_hit, const char* pool,
                                   size_t pool_stride) {
  if (!ffn_fused_ok(wfmt, H, I) || flags == nullptr || (seq == 0 && seq_dev == nullptr)) return hipErrorInvalidValue;
  if (max_items == 0) return hipSuccess;
  if (pool == nullptr)
    return fused_kernel(wfmt, DevHits{{n_items, items}}, x, perm_src, max_items, slot_base, slot_stride, H, I, hbuf, y,
                        flags, seq, seq_dev, s);
  return fused_kernel(wfmt, DevWork{{n_items, items}, n_hit, pool, pool_stride}, x, perm_src, max_items, slot_base,
                      slot_stride, H, I, hbuf, y, flags, seq, seq_dev, s);
}

bool ffn_combine_ok(int wfmt, int H, int I, int max_items, int T, int k) {
  return wfmt == 1 && H % 16 == 0 && I % 512 == 0 && I / 512 <= kU / 2 && max_items <= kFuseItems && T >= 1 &&
         T <= 16 && k >= 1 && T * k <= kFuseRows;
}

namespace {

template <typename W>
hipError_t ffn_combine_kernels(const W& wk, const void* x, const int32_t* perm_src, int max_items, int T,
                               const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y_perm,
                               const int32_t* n_active, const int32_t* perm_pos, const float* topk_w, int k, void* out,
                               bool out_bf16, hipStream_t s) {
  const BlobLayout L = blob_layout(1, H, I);
  hipLaunchKernelGGL(ffn1_decode_bf16<W>, dim3(max_items * (I / 8)), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                     perm_src, wk, slot_base, slot_stride, H, I, static_cast<uint16_t*>(hbuf));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint16_t* h = static_cast<const uint16_t*>(hbuf);
  const dim3 grid(H / 16), block(64 * kFuseWaves);
  switch (I / 512) {
    case 1:
      hipLaunchKernelGGL((ffn2_combine_bf16<W, 1>), grid, block, 0, s, h, wk, slot_base, slot_stride, L.p2, H, I,
                         y_perm, n_active, perm_pos, topk_w, T, k, out, (int)out_bf16);
      break;
    case 2:
      hipLaunchKernelGGL((ffn2_combine_bf16<W, 2>), grid, block, 0, s, h, wk, slot_base, slot_stride, L.p2, H, I,
                         y_perm, n_active, perm_pos, topk_w, T, k, out, (int)out_bf16);
      break;
    case 3:
      hipLaunchKernelGGL((ffn2_combine_bf16<W, 3>), grid, block, 0, s, h, wk, slot_base, slot_stride, L.p2, H, I,
                         y_perm, n_active, perm_pos, topk_w, T, k, out, (int)out_bf16);
      break;
    default:
      hipLaunchKernelGGL((ffn2_combine_bf16<W, 4>), grid, block, 0, s, h, wk, slot_base, slot_stride, L.p2, H, I,
                         y_perm, n_active, perm_pos, topk_w, T, k, out, (int)out_bf16);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_decode_combine(const void* x, const int32_t* perm_src, const int32_t* n_items, const int4* items,
                                     int max_items, int T, const char* slot_base, size_t slot_stride, int H, int I,
                                     void* hbuf, float* y_perm, const int32_t* n_active, const int32_t* perm_pos,
                                     const float* topk_w, int k, void* out, bool out_bf16, hipStream_t s,
                                     const int32_t* n_hit, const char* pool, size_t pool_stride) {
  if (!ffn_combine_ok(1, H, I, max_items, T, k)) return hipErrorInvalidValue;
  if (pool == nullptr)
    return ffn_combine_kernels(DevHits{{n_items, items}}, x, perm_src, max_items, T, slot_base, slot_stride, H, I,
                               hbuf, y_perm, n_active, perm_pos, topk_w, k, out, out_bf16, s);
  return ffn_combine_kernels(DevWork{{n_items, items}, n_hit, pool, pool_stride}, x, perm_src, max_items, T, slot_base,
                             slot_stride, H, I, hbuf, y_perm, n_active, perm_pos, topk_w, k, out, out_bf16, s);
}

hipError_t launch_ffn_prefill(const void* x, const int32_t* perm_src, WorkArgs& wa, const char* slot_base,
                              size_t slot_stride, int H, int I, void* hbuf, float* y, hipStream_t s) {
  if (wa.n == 0) return hipSuccess;
  const BlobLayout L = blob_layout(1, H, I);
  int tot = 0;
  for (int i = 0; i < wa.n; ++i) {
    wa.tile_prefix[i] = tot;
    tot += (wa.item[i].z + kGemmBM - 1) / kGemmBM;
  }
  wa.tile_prefix[wa.n] = tot;
  wa.total_tiles = tot;
  if (tot == 0) return hipSuccess;
  hipLaunchKernelGGL(ffn_gemm_bf16<1>, dim3(tot * ((2 * I) / kGemmBN)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), perm_src, wa, slot_base, slot_stride, L.p1, 2 * I, H, H, I,
                     static_cast<uint16_t*>(hbuf), y, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ffn_gemm_bf16<2>, dim3(tot * (H / kGemmBN)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(hbuf), perm_src, wa, slot_base, slot_stride, L.p2, H, I, H, I,
                     static_cast<uint16_t*>(hbuf), y, nullptr);
  return hipGetLastError();
}

int router_gemm_splits(int T, int H, int E) { return gemm2_supported(E, H) ? router_gemm2_splits(T, H, E) : 1; }

hipError_t launch_router_gemm(const void* x, const void* wrt, int T, int H, int E, float* partial, int nsplit,
                              hipStream_t s) {
  if (gemm2_supported(E, H)) return launch_router_gemm2(x, wrt, T, H, E, partial, nsplit, s);
  if (nsplit != 1) return hipErrorInvalidValue;
  WorkArgs wa;
  memset(&wa, 0, sizeof wa);
  wa.n = 1;
  wa.item[0] = make_int4(0, 0, T, 0);
  wa.tile_prefix[0] = 0;
  wa.tile_prefix[1] = (T + kGemmBM - 1) / kGemmBM;
  wa.total_tiles = wa.tile_prefix[1];
  hipLaunchKernelGGL(ffn_gemm_bf16<0>, dim3(wa.total_tiles * (E / kGemmBN)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), nullptr, wa, static_cast<const char*>(wrt), 0, 0, E, H, H, 0,
                     nullptr, partial, nullptr);
  return hipGetLastError();
}

}  // namespace moe
