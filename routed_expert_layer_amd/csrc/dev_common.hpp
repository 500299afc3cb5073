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
__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

// (x & m) | c in one instruction (the compiler emits an and and an or). At
// most one scalar operand per vector instruction: the mask comes from a
// scalar register, the constant from a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// Eight int4 codes (nibble order k0,k2,k4,k6,k1,k3,k5,k7, stored as q+8) to
// eight fp16 values in k order. A nibble n placed in the low mantissa bits of
// 1024 (0x6400 | n) is 1024 + n exactly, and 1024 + n - 1032 = q. A nibble
// left four bits up (0x6400 | n << 4) is 1024 + 16 n, and (1024 + 16 n) / 16
// - 72 = q, one fused multiply-add whose exact result needs no rounding; so
// of the four nibble pairs of a word only the upper two need a shift (one,
// shared), and each pair costs one and-or and one packed fp16 operation.
__device__ __forceinline__ u32x4_t int4x8_to_f16x8(uint32_t w) {
  const uint32_t magic = 0x64006400u;
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t hi = w >> 8;
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, and_or(w, 0x000F000Fu, magic)) - off);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, and_or(w, 0x00F000F0u, magic)),
                                                                sixteenth, off16));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, and_or(hi, 0x000F000Fu, magic)) - off);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, and_or(hi, 0x00F000F0u, magic)),
                                                                sixteenth, off16));
  return r;
}

}  // namespace moe
