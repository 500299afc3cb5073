// Device helpers shared by the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)v);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// (x & m) | c in one instruction (the compiler emits an and and an or). At
// most one scalar operand per vector instruction: the mask comes from a
// scalar register, the constant from a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// Eight int4 codes (nibble order k0,k2,k4,k6,k1,k3,k5,k7, nibble n = q + 8) to eight bf16 values
// 1 + n/16 in k order: nibble n placed in the top four mantissa bits of 1.0
// (0x3F80 | n << 3) is 1 + n/16 exactly, so one shift and one and-or per pair
// of codes and no arithmetic. Since 1 + n/16 = 1.5 + q/16, a sum over a block
// of K is sum(q x) = 16 sum((1 + n/16) x) - 24 sum(x).
__device__ __forceinline__ u32x4_t int4x8_to_bf16x8_biased(uint32_t w) {
  const uint32_t one = 0x3F803F80u, mask = 0x00780078u;
  u32x4_t r;
  r[0] = and_or(w << 3, mask, one);   // nibbles 0, 4: k0, k1
  r[1] = and_or(w >> 1, mask, one);   // nibbles 1, 5: k2, k3
  r[2] = and_or(w >> 5, mask, one);   // nibbles 2, 6: k4, k5
  r[3] = and_or(w >> 9, mask, one);   // nibbles 3, 7: k6, k7
  return r;
}

// Rank of this thread's flag among the set flags of a block of NW waves (in
// thread order) and their total; `cnt` is LDS scratch of NW ints. Every
// thread of the block must call it.
template <int NW>
__device__ __forceinline__ int block_flag_rank(bool f, int* cnt, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) cnt[wv] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    const int c = cnt[w];
    base += w < wv ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + below;
}

}  // namespace moe
