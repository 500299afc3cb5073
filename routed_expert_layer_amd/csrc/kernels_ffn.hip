// Grouped SwiGLU expert FFN: y = (silu(x W1) * (x W3)) W2 for each listed
// expert over its group of rows.
//
// Decode (few rows per expert) is bound by streaming the expert's weights
// from HBM: the matrix-vector kernels give each workgroup one 16-row tile of
// a weight matrix, split its K range over four waves, and feed every 1 KiB
// weight fragment straight from a coalesced global load into a 16x16x32
// matrix-core instruction whose other operand holds the (<= 16) tokens.
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
// With `pool` set, items from *n_hit on are misses: their blob is read from the
// host pool (pool + expert * pool_stride, device-visible pinned memory) and
// written through into their slot, so the fill and the FFN are one pass.
struct DevWork {
  const int32_t* n;
  const int4* items;
  const int32_t* n_hit;
  const char* pool;
  size_t pool_stride;
  __device__ __forceinline__ bool get(int i, int4& it) const {
    if (i >= *n) return false;
    it = items[i];
    return true;
  }
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
};

__device__ __forceinline__ void st16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

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

// One wave's share of a tile: the sum over fragments [c0, c1) (1 KiB apart
// from wp) of each fragment times the activation fragment at ar + 32c. With
// WT every weight fragment is also stored at the same offset from fp (the
// write-through of a miss); the stores follow each batch's loads, and the
// variant without them keeps its loads free to move.
template <bool WT>
__device__ __forceinline__ f32x4_t bf16_wave_dot(const char* wp, char* fp, const uint16_t* ar, bool valid, int c0,
                                                 int c1) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int c = c0;
  for (; c + kU <= c1; c += kU) {
    u32x4_t a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      a[u] = ld16_nt(wp + (size_t)(c + u) * 1024);
      b[u] = valid ? ld16(ar + (c + u) * 32) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (WT) {
#pragma unroll
      for (int u = 0; u < kU; ++u) st16(fp + (size_t)(c + u) * 1024, a[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc = mfma_bf16(a[u], b[u], acc);
  }
  for (; c < c1; ++c) {
    const u32x4_t a = ld16_nt(wp + (size_t)c * 1024);
    const u32x4_t b = valid ? ld16(ar + c * 32) : u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (WT) st16(fp + (size_t)c * 1024, a);
    acc = mfma_bf16(a, b, acc);
  }
  return acc;
}

// Gate/up: workgroup = one 16-row tile of P1 (8 gate + 8 up columns) of one
// item; wave w reduces fragments [KC*w/4, KC*(w+1)/4).
template <typename W>
__global__ __launch_bounds__(256) void ffn1_decode_bf16(const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ perm_src, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride, int H,
                                                        int I, uint16_t* __restrict__ hbuf) {
  const int NT = I / 8;
  const int item = blockIdx.x / NT, tile = blockIdx.x - item * NT;
  int4 it;
  if (!wk.get(item, it)) return;
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
    const f32x4_t acc =
        fp ? bf16_wave_dot<true>(wp, fp, xr, valid, c0, c1) : bf16_wave_dot<false>(wp, nullptr, xr, valid, c0, c1);
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && valid) {
      const f32x4_t s = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
      const int i0 = 8 * tile + 2 * (lane >> 4);
      const uint32_t packed =
          (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16);
      *reinterpret_cast<uint32_t*>(hbuf + (size_t)(it.y + m) * I + i0) = packed;
    }
    __syncthreads();
  }
}

// Down projection: workgroup = one 16-row tile of P2 (16 output columns).
template <typename W>
__global__ __launch_bounds__(256) void ffn2_decode_bf16(const uint16_t* __restrict__ hbuf, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride,
                                                        size_t p2_off, int H, int I, float* __restrict__ y) {
  const int NT = H / 16;
  const int item = blockIdx.x / NT, tile = blockIdx.x - item * NT;
  int4 it;
  if (!wk.get(item, it)) return;
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
    const f32x4_t acc =
        fp ? bf16_wave_dot<true>(wp, fp, hr, valid, c0, c1) : bf16_wave_dot<false>(wp, nullptr, hr, valid, c0, c1);
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && valid) {
      const f32x4_t s = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
      *reinterpret_cast<f32x4_t*>(y + (size_t)(it.y + m) * H + 16 * tile + 4 * (lane >> 4)) = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// int4 decode kernels (x and the SwiGLU product in fp16, codes exact in fp16,
// one fp16 scale per 128-row block applied to that block's partial sum).
// ---------------------------------------------------------------------------

// Gathered activations, converted to fp16: xg[r, :] = fp16(x[perm_src[r], :]).
template <typename W>
__global__ __launch_bounds__(256) void gather_f16_kernel(const uint16_t* __restrict__ x,
                                                         const int32_t* __restrict__ perm_src, const W wk,
                                                         int H, uint16_t* __restrict__ xg) {
  int4 it;
  if (!wk.get(blockIdx.y, it)) return;
  const int H8 = H / 8;
  for (int idx = blockIdx.x * 256 + threadIdx.x; idx < it.z * H8; idx += gridDim.x * 256) {
    const int m = idx / H8, c = idx - (idx / H8) * H8;
    const u32x4_t v = ld16(x + (size_t)perm_src[it.y + m] * H + 8 * c);
    u32x4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float lo = __uint_as_float(v[p] << 16), hi = __uint_as_float(v[p] & 0xFFFF0000u);
      o[p] = (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
    }
    *reinterpret_cast<u32x4_t*>(xg + (size_t)(it.y + m) * H + 8 * c) = o;
  }
}

// One 128-wide K block of one 16-row tile: four fp16 matrix-core products of
// the dequantised codes a with the activation fragments b, scaled by the tile
// rows' block scales (four fp16 in sc0, sc1) and added to acc.
__device__ __forceinline__ void int4_tile_mac(const u32x4_t& a, uint32_t sc0, uint32_t sc1, const u32x4_t (&b)[4],
                                              f32x4_t& acc) {
  f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) t = mfma_f16(int4x8_to_f16x8(a[j]), b[j], t);
  acc[0] = fmaf(t[0], f16_bits_to_f32(sc0 & 0xFFFFu), acc[0]);
  acc[1] = fmaf(t[1], f16_bits_to_f32(sc0 >> 16), acc[1]);
  acc[2] = fmaf(t[2], f16_bits_to_f32(sc1 & 0xFFFFu), acc[2]);
  acc[3] = fmaf(t[3], f16_bits_to_f32(sc1 >> 16), acc[3]);
}

// Shared body of both int4 projections. A block owns kR consecutive 16-row
// tiles of one expert; its four waves split K, and each wave applies every
// activation fragment it loads to all kR tiles (one activation load per kR
// KiB of codes). Partial sums meet in LDS; wave w finishes tile w.
// act: fp16 activations [rows, K] (gathered x or h); the finished 16 x 16
// tile sums go to `emit(tile, m, sum)`. With WT every code and scale loaded
// is also stored at the same offset from qf_base / sf_base (the write-through
// of a miss), after each K block's loads.
constexpr int kR = 4;
template <bool WT, typename Emit>
__device__ __forceinline__ void int4_decode_tiles(const uint16_t* __restrict__ act, const int4 it, int K,
                                                  const char* q_base, const char* s_base, char* qf_base,
                                                  char* sf_base, int tile0, Emit emit) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KG = K / 128;
  const int g0 = (KG * wave) >> 2, g1 = (KG * (wave + 1)) >> 2;
  const int kq = (lane >> 4) * 8;
  __shared__ f32x4_t red[4][kR][64];
  for (int m0 = 0; m0 < it.z; m0 += 16) {
    const int m = m0 + (lane & 15);
    const bool valid = m < it.z;
    const uint16_t* ar = act + (size_t)(it.y + (valid ? m : 0)) * K + kq;
    f32x4_t acc[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int g = g0; g < g1; ++g) {
      u32x4_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = valid ? ld16(ar + 128 * g + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t a[kR];
      uint32_t sc0[kR], sc1[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const size_t blk = (size_t)(tile0 + r) * KG + g;
        a[r] = ld16_nt(q_base + blk * 1024 + lane * 16);
        // The four fp16 scales are read as two 32-bit words and widened one by
        // one (a two-element fp16 vector view of the 64-bit load was
        // miscompiled into mixed-precision FMAs that all read the first word).
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(s_base + blk * 32 + (lane >> 4) * 8);
        sc0[r] = sp[0];
        sc1[r] = sp[1];
      }
      if constexpr (WT) {  // codes by every lane, each 8-byte scale group by one lane
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const size_t blk = (size_t)(tile0 + r) * KG + g;
          st16(qf_base + blk * 1024 + lane * 16, a[r]);
          if ((lane & 15) == 0) {
            uint32_t* sf = reinterpret_cast<uint32_t*>(sf_base + blk * 32 + (lane >> 4) * 8);
            sf[0] = sc0[r];
            sf[1] = sc1[r];
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) int4_tile_mac(a[r], sc0[r], sc1[r], b, acc[r]);
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
__global__ __launch_bounds__(256) void ffn1_decode_int4(const uint16_t* __restrict__ xg, const W wk,
                                                        const char* __restrict__ slot_base, size_t slot_stride,
                                                        size_t p1s_off, int H, int I, uint16_t* __restrict__ hbuf) {
  const int NB = I / 8 / kR;  // blocks per expert
  const int item = blockIdx.x / NB, tile0 = (blockIdx.x - item * NB) * kR;
  int4 it;
  if (!wk.get(item, it)) return;
  char* fill;
  const char* blob = wk.src(item, it, slot_base, slot_stride, fill);
  const int lane = threadIdx.x & 63;
  const auto emit = [&](int tile, int m, const f32x4_t& s) {
    const int i0 = 8 * tile + 2 * (lane >> 4);
    const uint32_t packed =
        (uint32_t)f32_to_f16_bits(silu(s[0]) * s[1]) | ((uint32_t)f32_to_f16_bits(silu(s[2]) * s[3]) << 16);
    *reinterpret_cast<uint32_t*>(hbuf + (size_t)(it.y + m) * I + i0) = packed;
  };
  if (fill)
    int4_decode_tiles<true>(xg, it, H, blob, blob + p1s_off, fill, fill + p1s_off, tile0, emit);
  else
    int4_decode_tiles<false>(xg, it, H, blob, blob + p1s_off, nullptr, nullptr, tile0, emit);
}

template <typename W>
__global__ __launch_bounds__(256) void ffn2_decode_int4(const uint16_t* __restrict__ hbuf, const W wk,
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
  const auto emit = [&](int tile, int m, const f32x4_t& s) {
    *reinterpret_cast<f32x4_t*>(y + (size_t)(it.y + m) * H + 16 * tile + 4 * (lane >> 4)) = s;
  };
  if (fill)
    int4_decode_tiles<true>(hbuf, it, I, blob + p2_off, blob + p2s_off, fill + p2_off, fill + p2s_off, tile0, emit);
  else
    int4_decode_tiles<false>(hbuf, it, I, blob + p2_off, blob + p2s_off, nullptr, nullptr, tile0, emit);
}

// ---------------------------------------------------------------------------
// MXFP4 decode kernels (bf16 activations; every FP4 code times its power-of-two
// block scale is exact in bf16, so the weights enter bf16 matrix-core
// instructions exactly and the result equals a bf16-weight product with the
// dequantised weights).
// ---------------------------------------------------------------------------

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
template <bool WT, typename Row, typename Emit>
__device__ __forceinline__ void mxfp4_decode_tiles(Row act_row, const int4 it, int K, const char* q_base,
                                                   const char* s_base, char* qf_base, char* sf_base, int tile0,
                                                   Emit emit) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KG = K / 128;
  const int g0 = (KG * wave) >> 2, g1 = (KG * (wave + 1)) >> 2;
  const int kq = (lane >> 4) * 8;
  __shared__ f32x4_t red[4][kR][64];
  for (int m0 = 0; m0 < it.z; m0 += 16) {
    const int m = m0 + (lane & 15);
    const bool valid = m < it.z;
    const uint16_t* ar = act_row(valid ? m : 0) + kq;
    f32x4_t acc[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int g = g0; g < g1; ++g) {
      u32x4_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = valid ? ld16(ar + 128 * g + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
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
      }
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[r] = mfma_bf16(fp4x8_to_bf16x8(a[r][j], e8m0_to_f32(sc[r] >> (8 * j))), b[j], acc[r]);
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
                          const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, void* xg, float* y,
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
  hipLaunchKernelGGL(gather_f16_kernel<W>, dim3(4, n_items), dim3(256), 0, s, static_cast<const uint16_t*>(x), perm_src,
                     wk, H, static_cast<uint16_t*>(xg));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ffn1_decode_int4<W>, dim3(n_items * (I / 8 / kR)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(xg), wk, slot_base, slot_stride, L.p1s, H, I,
                     static_cast<uint16_t*>(hbuf));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ffn2_decode_int4<W>, dim3(n_items * (H / 16 / kR)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(hbuf), wk, slot_base, slot_stride, L.p2, L.p2s, H, I, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_decode(int wfmt, const void* x, const int32_t* perm_src, const WorkArgs& wa,
                             const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, void* xg, float* y,
                             hipStream_t s) {
  if (wa.n == 0) return hipSuccess;
  int max_rows = 0;
  for (int i = 0; i < wa.n; ++i) max_rows = wa.item[i].z > max_rows ? wa.item[i].z : max_rows;
  return decode_kernels(wfmt, x, perm_src, ArgWork{wa}, wa.n, max_rows, slot_base, slot_stride, H, I, hbuf, xg, y, s);
}

hipError_t launch_ffn_decode_dev(int wfmt, const void* x, const int32_t* perm_src, const int32_t* n_items,
                                 const int4* items, int max_items, int max_rows, const char* slot_base,
                                 size_t slot_stride, int H, int I, void* hbuf, void* xg, float* y, hipStream_t s,
                                 const int32_t* n_hit, const char* pool, size_t pool_stride) {
  if (max_items == 0) return hipSuccess;
  if (wfmt == 0 && pool != nullptr) return hipErrorInvalidValue;  // the fp32 kernels do not write through
  return decode_kernels(wfmt, x, perm_src, DevWork{n_items, items, n_hit, pool, pool_stride}, max_items, max_rows,
                        slot_base, slot_stride, H, I, hbuf, xg, y, s);
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
