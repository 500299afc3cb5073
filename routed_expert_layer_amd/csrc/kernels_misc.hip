// Weighted combine and expert-blob packing.
#include "dev_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// out[t, :] = sum_j w[t,j] * y_perm[perm_pos[t,j], :], j ascending, fp32.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ perm_pos,
                                                      const float* __restrict__ w, int T, int k, int H,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if ((H & 3) == 0 && k <= 8) {
    // every row position and weight first, then every row load, so the k
    // loads of a thread are in flight together; the sum keeps the order below
    int p[8];
    float wj[8];
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        p[j] = perm_pos[(size_t)t * k + j];
        wj[j] = w[(size_t)t * k + j];
      }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) v[j] = *reinterpret_cast<const float4*>(y + (size_t)p[j] * H + n);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        acc.x = fmaf(wj[j], v[j].x, acc.x);
        acc.y = fmaf(wj[j], v[j].y, acc.y);
        acc.z = fmaf(wj[j], v[j].z, acc.z);
        acc.w = fmaf(wj[j], v[j].w, acc.w);
      }
  } else if ((H & 3) == 0) {
    for (int j = 0; j < k; ++j) {
      const int p = perm_pos[(size_t)t * k + j];
      const float wj = w[(size_t)t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(y + (size_t)p * H + n);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
  } else {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int p = perm_pos[(size_t)t * k + j];
      const float wj = w[(size_t)t * k + j];
      for (int c = 0; c < 4 && n + c < H; ++c) a[c] = fmaf(wj, y[(size_t)p * H + n + c], a[c]);
    }
    acc = make_float4(a[0], a[1], a[2], a[3]);
  }
  const float av[4] = {acc.x, acc.y, acc.z, acc.w};
  for (int c = 0; c < 4 && n + c < H; ++c) {
    if constexpr (OUT_BF16)
      reinterpret_cast<uint16_t*>(out)[(size_t)t * H + n + c] = f32_to_bf16(av[c]);
    else
      reinterpret_cast<float*>(out)[(size_t)t * H + n + c] = av[c];
  }
}

// Fragment order of a [K, N] row-major bf16 matrix taken by columns: row
// tile t holds columns 16t..16t+15; one thread per 16-byte chunk.
__global__ void pack_frag_kernel(const uint16_t* __restrict__ W, int K, int N, char* __restrict__ dst) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KC = K / 32;
  if (q >= (size_t)(N / 16) * KC * 64) return;
  const int l = (int)(q % 64), c = (int)((q / 64) % KC), t = (int)(q / (64 * (size_t)KC));
  const int n = 16 * t + (l % 16);
  const int kb = 32 * c + 8 * (l / 16);
  uint16_t v[8];
  for (int j = 0; j < 8; ++j) v[j] = W[(size_t)(kb + j) * N + n];
  *reinterpret_cast<uint4*>(dst + q * 16) = *reinterpret_cast<uint4*>(v);
}

// Gate/up matrix of a bf16 blob (rows interleaved as p1_row_source says).
__global__ void pack_p1_bf16_kernel(const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W3, int H, int I,
                                    char* __restrict__ blob) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KC = H / 32;
  if (q >= (size_t)(2 * I / 16) * KC * 64) return;
  const int l = (int)(q % 64), c = (int)((q / 64) % KC), t = (int)(q / (64 * (size_t)KC));
  int mat, i;
  p1_row_source(16 * t + (l % 16), mat, i);
  const uint16_t* W = mat ? W3 : W1;
  const int kb = 32 * c + 8 * (l / 16);
  uint16_t v[8];
  for (int j = 0; j < 8; ++j) v[j] = W[(size_t)(kb + j) * I + i];
  *reinterpret_cast<uint4*>(blob + q * 16) = *reinterpret_cast<uint4*>(v);
}

__device__ __forceinline__ uint32_t pack_word(const int8_t* Q, int ld, int col, int k0) {
  // nibble p (p < 4) = code(k0 + 2p), nibble p + 4 = code(k0 + 2p + 1); code = q + 8
  uint32_t w = 0;
  for (int p = 0; p < 4; ++p) {
    const uint32_t even = (uint32_t)(Q[(size_t)(k0 + 2 * p) * ld + col] + 8) & 0xFu;
    const uint32_t odd = (uint32_t)(Q[(size_t)(k0 + 2 * p + 1) * ld + col] + 8) & 0xFu;
    w |= even << (4 * p);
    w |= odd << (4 * (p + 4));
  }
  return w;
}

// int4 blob: codes one thread per 16-byte chunk, then scales.
__global__ void pack_int4_kernel(const int8_t* __restrict__ Q1, const int8_t* __restrict__ Q3,
                                 const int8_t* __restrict__ Q2, const uint16_t* __restrict__ S1,
                                 const uint16_t* __restrict__ S3, const uint16_t* __restrict__ S2, int H, int I,
                                 char* __restrict__ blob, size_t p1s, size_t p2, size_t p2s) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KG1 = H / 128, KG2 = I / 128;
  const size_t c1 = (size_t)(2 * I / 16) * KG1 * 64;       // P1 code chunks
  const size_t c2 = (size_t)(H / 16) * KG2 * 64;           // P2 code chunks
  const size_t s1n = (size_t)(2 * I / 16) * KG1 * 16;      // P1 scales
  const size_t s2n = (size_t)(H / 16) * KG2 * 16;          // P2 scales
  if (q < c1) {
    const int l = (int)(q % 64), g = (int)((q / 64) % KG1), t = (int)(q / (64 * (size_t)KG1));
    int mat, i;
    p1_row_source(16 * t + (l % 16), mat, i);
    const int8_t* Q = mat ? Q3 : Q1;
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) w[j] = pack_word(Q, I, i, 128 * g + 32 * j + 8 * (l / 16));
    *reinterpret_cast<uint4*>(blob + q * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  size_t r = q - c1;
  if (r < c2) {
    const int l = (int)(r % 64), g = (int)((r / 64) % KG2), t = (int)(r / (64 * (size_t)KG2));
    const int n = 16 * t + (l % 16);
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) w[j] = pack_word(Q2, H, n, 128 * g + 32 * j + 8 * (l / 16));
    *reinterpret_cast<uint4*>(blob + p2 + r * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  r -= c2;
  if (r < s1n) {
    const int rr = (int)(r % 16), g = (int)((r / 16) % KG1), t = (int)(r / (16 * (size_t)KG1));
    int mat, i;
    p1_row_source(16 * t + rr, mat, i);
    const uint16_t* S = mat ? S3 : S1;
    reinterpret_cast<uint16_t*>(blob + p1s)[r] = S[(size_t)g * I + i];
    return;
  }
  r -= s1n;
  if (r < s2n) {
    const int rr = (int)(r % 16), g = (int)((r / 16) % KG2), t = (int)(r / (16 * (size_t)KG2));
    reinterpret_cast<uint16_t*>(blob + p2s)[r] = S2[(size_t)g * H + 16 * t + rr];
  }
}

// Eight FP4 codes of column `col`, rows k0..k0+7 of a [K, ld] uint8 code
// matrix, as nibbles in row order (nibble p = code of row k0 + p).
__device__ __forceinline__ uint32_t pack_fp4_word(const uint8_t* C, int ld, int col, int k0) {
  uint32_t w = 0;
  for (int p = 0; p < 8; ++p) w |= ((uint32_t)C[(size_t)(k0 + p) * ld + col] & 0xFu) << (4 * p);
  return w;
}

// MXFP4 blob: one thread per 16-byte code chunk, then one per 4-byte scale word.
__global__ void pack_mxfp4_kernel(const uint8_t* __restrict__ C1, const uint8_t* __restrict__ C3,
                                  const uint8_t* __restrict__ C2, const uint8_t* __restrict__ S1,
                                  const uint8_t* __restrict__ S3, const uint8_t* __restrict__ S2, int H, int I,
                                  char* __restrict__ blob, size_t p1s, size_t p2, size_t p2s) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KG1 = H / 128, KG2 = I / 128;
  const size_t c1 = (size_t)(2 * I / 16) * KG1 * 64;       // P1 code chunks
  const size_t c2 = (size_t)(H / 16) * KG2 * 64;           // P2 code chunks
  const size_t s1n = (size_t)(2 * I / 16) * KG1 * 16;      // P1 scale words
  const size_t s2n = (size_t)(H / 16) * KG2 * 16;          // P2 scale words
  if (q < c1) {
    const int l = (int)(q % 64), g = (int)((q / 64) % KG1), t = (int)(q / (64 * (size_t)KG1));
    int mat, i;
    p1_row_source(16 * t + (l % 16), mat, i);
    const uint8_t* C = mat ? C3 : C1;
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) w[j] = pack_fp4_word(C, I, i, 128 * g + 32 * j + 8 * (l / 16));
    *reinterpret_cast<uint4*>(blob + q * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  size_t r = q - c1;
  if (r < c2) {
    const int l = (int)(r % 64), g = (int)((r / 64) % KG2), t = (int)(r / (64 * (size_t)KG2));
    const int n = 16 * t + (l % 16);
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) w[j] = pack_fp4_word(C2, H, n, 128 * g + 32 * j + 8 * (l / 16));
    *reinterpret_cast<uint4*>(blob + p2 + r * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  r -= c2;
  if (r < s1n) {
    const int rr = (int)(r % 16), g = (int)((r / 16) % KG1), t = (int)(r / (16 * (size_t)KG1));
    int mat, i;
    p1_row_source(16 * t + rr, mat, i);
    const uint8_t* S = mat ? S3 : S1;
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j) w |= (uint32_t)S[(size_t)(4 * g + j) * I + i] << (8 * j);
    reinterpret_cast<uint32_t*>(blob + p1s)[r] = w;
    return;
  }
  r -= s1n;
  if (r < s2n) {
    const int rr = (int)(r % 16), g = (int)((r / 16) % KG2), t = (int)(r / (16 * (size_t)KG2));
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j) w |= (uint32_t)S2[(size_t)(4 * g + j) * H + 16 * t + rr] << (8 * j);
    reinterpret_cast<uint32_t*>(blob + p2s)[r] = w;
  }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* perm_pos, const float* w, int T, int k, int H,
                          void* out, bool out_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid(T, (H + 1023) / 1024);
  if (out_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, y_perm, perm_pos, w, T, k, H, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, y_perm, perm_pos, w, T, k, H, out);
  return hipGetLastError();
}

// Sets n bytes at p to 0xFF: 16-byte stores over the aligned body, single
// bytes for a ragged head and tail; fixed grid, grid-stride loop.
__global__ __launch_bounds__(256) void poison_kernel(char* __restrict__ p, size_t n) {
  const size_t head = (16 - (reinterpret_cast<uintptr_t>(p) & 15)) & 15;
  const size_t h = head < n ? head : n;
  const size_t body = (n - h) / 16;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)gridDim.x * blockDim.x;
  uint4* b = reinterpret_cast<uint4*>(p + h);
  for (size_t i = tid; i < body; i += stride) b[i] = make_uint4(~0u, ~0u, ~0u, ~0u);
  if (tid < h) p[tid] = (char)0xFF;
  const size_t tail0 = h + body * 16;
  if (tid < n - tail0) p[tail0 + tid] = (char)0xFF;
}

hipError_t launch_poison(void* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(poison_kernel, dim3(1024), dim3(256), 0, s, static_cast<char*>(p), n);
  return hipGetLastError();
}

hipError_t launch_pack_fragments(const void* W, int K, int N, void* dst, hipStream_t s) {
  const size_t n = (size_t)(N / 16) * (K / 32) * 64;
  hipLaunchKernelGGL(pack_frag_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(W), K, N, static_cast<char*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack(int wfmt, int H, int I, const void* W1, const void* W3, const void* W2, const void* s1,
                       const void* s3, const void* s2, void* blob, hipStream_t s) {
  const BlobLayout L = blob_layout(wfmt, H, I);
  const size_t HI = (size_t)H * I;
  char* b = static_cast<char*>(blob);
  if (wfmt == 0) {
    hipError_t e = hipMemcpyAsync(b, W1, HI * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(b + HI * 4, W3, HI * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(b + 2 * HI * 4, W2, HI * 4, hipMemcpyDeviceToDevice, s);
    return e;
  }
  if (wfmt == 1) {
    const size_t n1 = (size_t)(2 * I / 16) * (H / 32) * 64;
    hipLaunchKernelGGL(pack_p1_bf16_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(W1), static_cast<const uint16_t*>(W3), H, I, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_pack_fragments(W2, I, H, b + L.p2, s);
  }
  if (wfmt == 3) {  // MXFP4 (alignment padding between sections is never read)
    const size_t n = (size_t)(2 * I / 16) * (H / 128) * 64 + (size_t)(H / 16) * (I / 128) * 64 +
                     (size_t)(2 * I / 16) * (H / 128) * 16 + (size_t)(H / 16) * (I / 128) * 16;
    hipLaunchKernelGGL(pack_mxfp4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(W1), static_cast<const uint8_t*>(W3),
                       static_cast<const uint8_t*>(W2), static_cast<const uint8_t*>(s1),
                       static_cast<const uint8_t*>(s3), static_cast<const uint8_t*>(s2), H, I, b, L.p1s, L.p2,
                       L.p2s);
    return hipGetLastError();
  }
  // int4 (alignment padding between sections is never read)
  const size_t n = (size_t)(2 * I / 16) * (H / 128) * 64 + (size_t)(H / 16) * (I / 128) * 64 +
                   (size_t)(2 * I / 16) * (H / 128) * 16 + (size_t)(H / 16) * (I / 128) * 16;
  hipLaunchKernelGGL(pack_int4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const int8_t*>(W1), static_cast<const int8_t*>(W3), static_cast<const int8_t*>(W2),
                     static_cast<const uint16_t*>(s1), static_cast<const uint16_t*>(s3),
                     static_cast<const uint16_t*>(s2), H, I, b, L.p1s, L.p2, L.p2s);
  return hipGetLastError();
}

}  // namespace moe
