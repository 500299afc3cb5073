// Large-tile grouped GEMM for prefill on bf16 matrix cores.
//
// Block tile: 256 weight rows (16 fragment rows) x 128 or 256 tokens (8 or
// 16 fragment columns of 16 tokens) x 32 K per stage. Eight waves (two per
// SIMD), each accumulating 64 x 64 (4 x 4 accumulator fragments, 128-token
// tile) or 128 x 64 (8 x 4, 256-token tile); per stage a wave reads 8 or 12
// one-KiB fragments from LDS for 16 or 32 matrix-core instructions.
// Operands go straight from global memory into LDS in fragment order (the
// direct-to-LDS load of gfx950, one 1 KiB fragment per wave instruction, no
// register staging), through six (128-token tile) or four (256-token tile)
// LDS stages, all in flight; a wave reads the next stage's fragments into a
// second register set while its matrix-core instructions consume the current
// one; one barrier per stage. Weight fragments are contiguous
// in the expert blob (1 KiB per wave load); token rows are gathered through
// perm_src (gate/up), read in order (down projection) or taken from x (router).
// Blocks are grouped into super-tiles of 32 (8 token tiles x 4 weight tiles
// when the weight tiles allow) that the dispatcher sends to one XCD together.
#include <algorithm>
#include <cstring>
#include <type_traits>
#include <vector>

#include "dev_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 at their maxima).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and for lgkmcnt <= n only (vmcnt and expcnt at their maxima).
constexpr int lgkmcnt_only(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }

// One 16-byte chunk per lane from base + off (a wave-uniform base, a 32-bit
// lane offset) straight into the wave's 1 KiB at `lds` (lane l at lds + 16 l),
// through a raw buffer resource (dword 3 = 0x00020000 for byte-addressed
// loads on gfx950, no bounds check).
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t off, char* lds) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Adds the shader-clock cycles and 100 MHz real-time ticks since (c0, r0) to
// sums[0] and sums[1] (the clock diagnostic; one call per block).
__device__ __forceinline__ void record_clock(unsigned long long* sums, unsigned long long c0, unsigned long long r0) {
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  atomicAdd(sums, c1 - c0);
  atomicAdd(sums + 1, r1 - r0);
}

// Process-wide target of the clock diagnostic (nullptr: off).
unsigned long long* g_clock_sums = nullptr;

// The work list comes by value (WorkArgs) or from device memory (GemmTable);
// both have the same fields.
__device__ inline const WorkArgs& table_of(const WorkArgs& w) { return w; }
__device__ inline const GemmTable& table_of(const GemmTable* t) { return *t; }

// One block tile (super-tile `sidx`, slot `w` in it) of the kernel below.
template <int PHASE, int BM_T, typename Tab>
__device__ __forceinline__ void gemm2_tile(const uint16_t* __restrict__ bsrc, const int32_t* __restrict__ perm_src,
                                           const Tab& tab, const char* __restrict__ slot_base, size_t slot_stride,
                                           size_t mat_off, int N, int K, int H, int I, uint16_t* __restrict__ hout,
                                           float* __restrict__ yout, const float* __restrict__ bias,
                                           unsigned long long* __restrict__ clock_sums, const int sidx, const int w) {
  const unsigned long long c_start = __builtin_amdgcn_s_memtime(), r_start = __builtin_amdgcn_s_memrealtime();
  constexpr int BN_T = 16;
  constexpr int NS = BM_T == 16 ? 4 : 6;       // LDS stages of 32 K; NS - 1 in flight
  constexpr int WN = BM_T == 16 ? 8 : 4;       // weight fragment rows per wave
  constexpr int WM = 4;                        // token fragment columns per wave
  constexpr int WAVES_N = BN_T / WN;           // wave grid: WAVES_N x (BM_T / WM) = 8 waves
  static_assert(WAVES_N * (BM_T / WM) == 8, "wave grid");
  constexpr int FA = BN_T, FB = BM_T;          // fragments per stage
  constexpr int FPW = (FA + FB) / 8;           // fragment loads per wave per stage
  static_assert((FA + FB) % 8 == 0, "stage must split over the waves");
  constexpr int STAGE = (FA + FB) * 1024;
  __shared__ __attribute__((aligned(1024))) char lds[NS][STAGE];

  // Super-tile schedule: 32 consecutive slots of one XCD (blocks b with the
  // same b % 8) form a super-tile of GM token tiles x GN weight tiles of one
  // expert, so the blocks that run together on an XCD share their operands in
  // its L2 while they advance through K at the same pace.
  const auto& wa = table_of(tab);
  const int NTB = N / (16 * BN_T);
  int lo = 0, hi = wa.n - 1;           // item with tile_prefix[item] <= sidx < tile_prefix[item + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wa.tile_prefix[mid] <= sidx) lo = mid; else hi = mid - 1;
  }
  const int item = lo;
  const int4 it = wa.item[item];
  const int GM = it.w & 0xFF, GN = it.w >> 8;  // this expert's super-tile shape
  if (w >= GM * GN) return;
  const int ls = sidx - wa.tile_prefix[item];
  const int ngroups = NTB / GN;
  const int mt = (ls / ngroups) * GM + w / GN;
  const int nt = (ls % ngroups) * GN + (w % GN);
  if (mt * 16 * BM_T >= it.z) return;  // past the expert's last token tile
  // the thread index passes through an empty asm so that nothing derived from it is hoisted out of the
  // kernel's loop over tiles (live across the whole tile, it would cost registers)
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int wn = wave % WAVES_N, wm = wave / WAVES_N;
  const int KC = K / 32;
  const int ldb = (PHASE == 2) ? I : H;
  // The router (PHASE 0) runs split over K: item.x is the split index, K the
  // split's length; its weight row tiles span all H / 32 chunks.
  const int KCW = (PHASE == 0) ? ldb / 32 : KC;
  const int koff = (PHASE == 0) ? it.x * KC : 0;

  // This wave loads stage fragments f = wave + 8q (q < FPW): weight fragment
  // row tile f for q < FA / 8, token column f - FA after. Loads are
  // buffer-addressed (a wave-uniform base plus a 32-bit lane offset): a flat
  // global -> LDS load would count as a pending flat LDS access and make the
  // compiler wait for every LDS read before the first matrix-core
  // instruction. Lane offsets exclude the K step; tokens past the group read
  // a valid row (their columns of the product are never stored).
  static_assert(FA % 8 == 0, "weight and token loads split at a fixed q");
  constexpr int QW = FA / 8;  // weight loads per wave per stage
  const char* wbase = slot_base + (size_t)it.x * slot_stride + mat_off;
  uint32_t off[FPW];
  uint32_t kstep[FPW];  // bytes per 32-wide K step
#pragma unroll
  for (int q = 0; q < FPW; ++q) {
    const int f = wave + 8 * q;
    if (q < QW) {
      off[q] = (uint32_t)(((nt * BN_T + f) * KCW + koff) * 1024 + lane * 16);
      kstep[q] = 1024;
    } else {
      int mloc = mt * (16 * BM_T) + (f - FA) * 16 + (lane & 15);
      if (mloc >= it.z) mloc = it.z - 1;
      if constexpr (PHASE == 2) {
        // h in fragment order: row r, 32-wide K chunk c at ((r/16) * KC + c) KiB
        const uint32_t row = (uint32_t)(it.y + mloc);
        off[q] = (row >> 4) * (uint32_t)KC * 1024u + ((row & 15) + 16 * (lane >> 4)) * 16;
        kstep[q] = 1024;
      } else {
        const uint32_t row = (PHASE == 1) ? (uint32_t)perm_src[it.y + mloc] : (uint32_t)(it.y + mloc);
        off[q] = (row * (uint32_t)ldb + (uint32_t)koff * 32 + (lane >> 4) * 8) * 2;
        kstep[q] = 64;
      }
    }
  }
  // Stage `stage` -> LDS buffer `buf`.
  auto issue = [&](int stage, int buf) {
    char* base = lds[buf];
#pragma unroll
    for (int q = 0; q < FPW; ++q)
      buffer_load_lds16(q < QW ? static_cast<const void*>(wbase) : static_cast<const void*>(bsrc),
                        off[q] + (uint32_t)stage * kstep[q], base + (wave + 8 * q) * 1024);
  };

  f32x4_t acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Frags {
    u32x4_t a[WN], b[WM];
  };
  // The K loop is instantiated for JM = the number of this wave's token
  // fragments that hold at least one row of the group (0 .. WM, uniform per
  // wave): fragments wholly past the group get no LDS reads and no
  // matrix-core work, which lowers the power drawn by partial tiles (a
  // 96-row group in a 128-token tile, the last tile of a large group, small
  // groups). The products kept are the same instructions in the same order,
  // so the results do not change.
  auto k_loop = [&](auto jm_const) {
    constexpr int JM = decltype(jm_const)::value;
    auto read_stage = [&](int kt, Frags& f) {
      const char* b = lds[kt % NS];
#pragma unroll
      for (int j = 0; j < JM; ++j)
        f.b[j] = *reinterpret_cast<const u32x4_t*>(b + (FA + wm * WM + j) * 1024 + lane * 16);
      if constexpr (JM > 0) {
#pragma unroll
        for (int i = 0; i < WN; ++i)
          f.a[i] = *reinterpret_cast<const u32x4_t*>(b + (wn * WN + i) * 1024 + lane * 16);
      }
    };
    auto compute = [&](const Frags& f) {
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < JM; ++j) acc[i][j] = mfma_bf16(f.a[i], f.b[j], acc[i][j]);
    };

  // All NS buffers are in flight. In step kt a wave computes on stage kt's
  // fragments (read into registers during step kt - 1) while it reads stage
  // kt + 1's, so LDS latency hides behind matrix-core work; after the step's
  // barrier (every wave's loads of stage kt + 1 have landed and every wave
  // has finished reading stage kt) stage kt's buffer is refilled with stage
  // kt + NS. The read past the last stage repeats the last one (results
  // unused), so the reads and the matrix-core instructions of a step form
  // one basic block for any K and the compiler can interleave them.
    auto step = [&](int kt, Frags& cur, Frags& nxt) {
      // this wave's loads of stage kt + 1 landed: at most the stages kt + 2 ..
      // kt + NS - 1 still in flight, or, near the end where fewer were
      // issued, none
      if (kt + NS - 1 < KC) {
        __builtin_amdgcn_s_waitcnt(vmcnt_only(FPW * (NS - 2)));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      }
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));  // and its reads of stage kt completed
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + NS < KC) issue(kt + NS, kt % NS);
      read_stage(min(kt + 1, KC - 1), nxt);
      compute(cur);
      // one LDS read, then a share of the matrix-core instructions, in turn
      // (no priority changes in between: they would fence the scheduler)
      if constexpr (JM > 0) {
#pragma unroll
        for (int q = 0; q < WN + JM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, (WN * JM) / (WN + JM), 0);
        }
      }
    };
    for (int s0 = 0; s0 < NS && s0 < KC; ++s0) issue(s0, s0);
    // stage 0 landed
    if (KC >= NS) {
      __builtin_amdgcn_s_waitcnt(vmcnt_only(FPW * (NS - 1)));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Frags f0, f1;
    read_stage(0, f0);
    int kt = 0;
    for (; kt + 1 < KC; kt += 2) {
      step(kt, f0, f1);
      step(kt + 1, f1, f0);
    }
    if (kt < KC) step(kt, f0, f1);
  };
  static_assert(WM == 4, "the dispatch below covers 0 .. 4 fragments");
  const int rows_here = it.z - (mt * 16 * BM_T + wm * WM * 16);
  const int jm = rows_here <= 0 ? 0 : min(WM, (rows_here + 15) / 16);
  switch (jm) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    default: k_loop(std::integral_constant<int, 4>{}); break;
  }
  if (clock_sums != nullptr && tid == 0) record_clock(clock_sums, c_start, r_start);

  // Epilogue.
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int mloc = mt * (16 * BM_T) + (wm * WM + j) * 16 + (lane & 15);
    if (mloc >= it.z) continue;
    const size_t row = (size_t)(it.y + mloc);
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int ntile = nt * BN_T + wn * WN + i;
      const f32x4_t s = acc[i][j];
      if constexpr (PHASE == 1) {
        // h is stored in the down projection's token-fragment order: row r,
        // columns 32c + 8g .. +7 at element ((r/16) * (I/32) + c) * 512 +
        // ((r % 16) + 16 g) * 8.
        const int i0 = 8 * ntile + 2 * (lane >> 4);
        const uint32_t packed =
            (uint32_t)f32_to_bf16(silu(s[0]) * s[1]) | ((uint32_t)f32_to_bf16(silu(s[2]) * s[3]) << 16);
        const size_t off = ((row >> 4) * (size_t)(I / 32) + (i0 >> 5)) * 512 + ((row & 15) + 16 * ((i0 & 31) >> 3)) * 8 +
                           (i0 & 7);
        *reinterpret_cast<uint32_t*>(hout + off) = packed;
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
        *reinterpret_cast<f32x4_t*>(yout + ((size_t)it.x * it.z + row) * N + n0) = o;  // split it.x's slab
      }
    }
  }
}

// Block b works on super-tiles (b / 256) * 8 + b % 8, then that plus 8 * (grid / 256), and so on, in slot
// (b / 8) % 32 of each: with a grid of exactly the planned rounds every block does one tile; a smaller grid (a
// multiple of 256) serves a work list planned on the device whose size the host does not know. Rounds keep the
// blocks of a super-tile on one XCD (the block index modulo 8 selects it). Every exit is uniform per block.
template <int PHASE, int BM_T, typename Tab>
__global__ __launch_bounds__(512, 1) void gemm2_bf16(const uint16_t* __restrict__ bsrc,
                                                        const int32_t* __restrict__ perm_src, const Tab tab,
                                                        const char* __restrict__ slot_base, size_t slot_stride,
                                                        size_t mat_off, int N, int K, int H, int I,
                                                        uint16_t* __restrict__ hout, float* __restrict__ yout,
                                                        const float* __restrict__ bias,
                                                        unsigned long long* __restrict__ clock_sums) {
  const int first = (int)(blockIdx.x >> 8), rounds = (int)(gridDim.x >> 8);
  const int total = table_of(tab).total_tiles;
  for (int r = first;; r += rounds) {
    const int sidx = r * 8 + (int)(blockIdx.x & 7);
    if (sidx >= total) break;
    if (r != first) __syncthreads();  // every wave is done with the previous tile's LDS stages
    gemm2_tile<PHASE, BM_T, Tab>(bsrc, perm_src, tab, slot_base, slot_stride, mat_off, N, K, H, I, hout, yout, bias,
                                 clock_sums, sidx, (int)((blockIdx.x >> 3) & 31));
  }
}

// ---------------------------------------------------------------------------
// The same grouped GEMM with MXFP4 weights (FP4 codes, one E8M0 scale per 32
// of K; the MOE_W_MXFP4 blob layout): 256 weight rows x 128 tokens per block
// and 128 K per stage (one 1 KiB code block per 16-row tile). Per stage each
// of the eight waves loads two code blocks, its two tiles' 64-byte scale
// blocks (eight lanes) and one 16-token fragment for each of the four 32-K
// sub-blocks, all straight into LDS (49 KiB per stage, three stages). Waves
// turn the codes of their four weight tiles into bf16 with the block scale
// folded in (exact) per 32-K sub-block and run 4 x 4 bf16 matrix-core
// products on them; the weight bytes crossing HBM and LDS are a quarter of
// the bf16 kernel's.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t mx_a_operand(uint32_t codes, uint32_t scale_byte) {
  const float sc = __uint_as_float((scale_byte & 0xFFu) << 23);
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
  return r;
}

// One block tile (super-tile `sidx`, slot `w` in it) of the kernel below.
template <int PHASE>
__device__ __forceinline__ void mxfp4_tile(const uint16_t* __restrict__ bsrc, const int32_t* __restrict__ perm_src,
                                           const GemmTable* __restrict__ tab, const char* __restrict__ slot_base,
                                           size_t slot_stride, size_t code_off, size_t scale_off, int N, int K, int I,
                                           int H, uint16_t* __restrict__ hout, float* __restrict__ yout,
                                           unsigned long long* __restrict__ clock_sums, const int sidx, const int w) {
  const unsigned long long c_start = __builtin_amdgcn_s_memtime(), r_start = __builtin_amdgcn_s_memrealtime();
  constexpr int BN_T = 16, BM_T = 8, NS = 3, WN = 4, WM = 4, WAVES_N = 4, KSUB = 4;
  constexpr int CODE = BN_T * 1024, SCL = BN_T * 64, TOK = BM_T * KSUB * 1024;
  constexpr int STAGE = CODE + SCL + TOK;
  constexpr int FPW = 7;  // per wave per stage: 2 code blocks, 1 scale load, 4 token fragments
  __shared__ __attribute__((aligned(1024))) char lds[NS][STAGE];

  const GemmTable& wa = *tab;
  const int NTB = N / (16 * BN_T);
  int lo = 0, hi = wa.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wa.tile_prefix[mid] <= sidx) lo = mid; else hi = mid - 1;
  }
  const int4 it = wa.item[lo];
  const int GM = it.w & 0xFF, GN = it.w >> 8;
  if (w >= GM * GN) return;
  const int ls = sidx - wa.tile_prefix[lo];
  const int ngroups = NTB / GN;
  const int mt = (ls / ngroups) * GM + w / GN;
  const int nt = (ls % ngroups) * GN + (w % GN);
  if (mt * 16 * BM_T >= it.z) return;
  // the thread index passes through an empty asm so that nothing derived from it is hoisted out of the
  // kernel's loop over tiles (live across the whole tile, it would cost registers)
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int wn = wave % WAVES_N, wm = wave / WAVES_N;
  const int KG = K / 128;  // stages
  const int KC = K / 32;
  const int ldb = (PHASE == 2) ? I : H;
  const char* blob = slot_base + (size_t)it.x * slot_stride;

  // load offsets at stage 0 and their step per stage
  uint32_t off[FPW], kstep[FPW];
#pragma unroll
  for (int q = 0; q < 2; ++q) {  // code blocks of weight tiles wave + 8q
    off[q] = (uint32_t)((((size_t)nt * BN_T + wave + 8 * q) * KG) * 1024 + lane * 16);
    kstep[q] = 1024;
  }
  // scale blocks of the same two tiles: lanes 0..3 tile `wave`, lanes 4..7 tile wave + 8
  off[2] = (uint32_t)((((size_t)nt * BN_T + wave + 8 * (lane >> 2 & 1)) * KG) * 64 + (lane & 3) * 16);
  kstep[2] = 64;
  {
    int mloc = mt * (16 * BM_T) + wave * 16 + (lane & 15);
    if (mloc >= it.z) mloc = it.z - 1;
    const uint32_t row = PHASE == 1 ? (uint32_t)perm_src[it.y + mloc] : (uint32_t)(it.y + mloc);
#pragma unroll
    for (int j = 0; j < KSUB; ++j) {  // token fragment (sub-block j, token tile `wave`)
      if constexpr (PHASE == 2) {
        off[3 + j] = (row >> 4) * (uint32_t)KC * 1024u + (uint32_t)j * 1024u + ((row & 15) + 16 * (lane >> 4)) * 16;
        kstep[3 + j] = 4096;
      } else {
        off[3 + j] = (row * (uint32_t)ldb + (uint32_t)j * 32 + (lane >> 4) * 8) * 2;
        kstep[3 + j] = 256;
      }
    }
  }
  auto issue = [&](int kt) {
    char* base = lds[kt % NS];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      buffer_load_lds16(blob + code_off, off[q] + (uint32_t)kt * kstep[q], base + (wave + 8 * q) * 1024);
    if (lane < 8) buffer_load_lds16(blob + scale_off, off[2] + (uint32_t)kt * kstep[2], base + CODE + wave * 128);
#pragma unroll
    for (int j = 0; j < KSUB; ++j)
      buffer_load_lds16(bsrc, off[3 + j] + (uint32_t)kt * kstep[3 + j], base + CODE + SCL + (j * BM_T + wave) * 1024);
  };

  f32x4_t acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int s0 = 0; s0 < NS - 1 && s0 < KG; ++s0) issue(s0);
  // As in the bf16 GEMM, the K loop is instantiated for JM = the number of
  // this wave's token fragments holding rows of the group: fragments past the
  // group get no LDS reads and no products, and a wave with none of the
  // group's rows converts no codes either. Kept products are unchanged.
  auto k_loop = [&](auto jm_const) {
    constexpr int JM = decltype(jm_const)::value;
    for (int kt = 0; kt < KG; ++kt) {
      if (kt + NS - 2 < KG) {
        __builtin_amdgcn_s_waitcnt(vmcnt_only(FPW * (NS - 2)));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + NS - 1 < KG) issue(kt + NS - 1);
      if constexpr (JM > 0) {
        const char* b = lds[kt % NS];
        u32x4_t codes[WN];
        uint32_t scl[WN];
#pragma unroll
        for (int i = 0; i < WN; ++i) {
          const int ta = wn * WN + i;  // weight tile of this wave
          codes[i] = *reinterpret_cast<const u32x4_t*>(b + ta * 1024 + lane * 16);
          scl[i] = *reinterpret_cast<const uint32_t*>(b + CODE + (ta & 7) * 128 + (ta >> 3) * 64 + (lane & 15) * 4);
        }
#pragma unroll
        for (int j = 0; j < KSUB; ++j) {
          u32x4_t bf[JM];
#pragma unroll
          for (int jj = 0; jj < JM; ++jj)
            bf[jj] =
                *reinterpret_cast<const u32x4_t*>(b + CODE + SCL + (j * BM_T + wm * WM + jj) * 1024 + lane * 16);
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int i = 0; i < WN; ++i) {
            const u32x4_t a = mx_a_operand(codes[i][j], scl[i] >> (8 * j));
#pragma unroll
            for (int jj = 0; jj < JM; ++jj) acc[i][jj] = mfma_bf16(a, bf[jj], acc[i][jj]);
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }
    }
  };
  static_assert(WM == 4, "the dispatch below covers 0 .. 4 fragments");
  const int rows_here = it.z - (mt * 16 * BM_T + wm * WM * 16);
  const int jm = rows_here <= 0 ? 0 : min(WM, (rows_here + 15) / 16);
  switch (jm) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    default: k_loop(std::integral_constant<int, 4>{}); break;
  }
  if (clock_sums != nullptr && threadIdx.x == 0) record_clock(clock_sums, c_start, r_start);

#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int mloc = mt * (16 * BM_T) + (wm * WM + j) * 16 + (lane & 15);
    if (mloc >= it.z) continue;
    const size_t row = (size_t)(it.y + mloc);
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int ntile = nt * BN_T + wn * WN + i;
      const f32x4_t sv = acc[i][j];
      if constexpr (PHASE == 1) {
        const int i0 = 8 * ntile + 2 * (lane >> 4);
        const uint32_t packed =
            (uint32_t)f32_to_bf16(silu(sv[0]) * sv[1]) | ((uint32_t)f32_to_bf16(silu(sv[2]) * sv[3]) << 16);
        const size_t o = ((row >> 4) * (size_t)(I / 32) + (i0 >> 5)) * 512 + ((row & 15) + 16 * ((i0 & 31) >> 3)) * 8 +
                         (i0 & 7);
        *reinterpret_cast<uint32_t*>(hout + o) = packed;
      } else {
        *reinterpret_cast<f32x4_t*>(yout + row * H + 16 * ntile + 4 * (lane >> 4)) = sv;
      }
    }
  }
}

// Rounds of super-tiles per block as for gemm2_bf16.
template <int PHASE>
__global__ __launch_bounds__(512, 1) void gemm_mxfp4(const uint16_t* __restrict__ bsrc,
                                                      const int32_t* __restrict__ perm_src,
                                                      const GemmTable* __restrict__ tab,
                                                      const char* __restrict__ slot_base, size_t slot_stride,
                                                      size_t code_off, size_t scale_off, int N, int K, int I,
                                                      int H, uint16_t* __restrict__ hout, float* __restrict__ yout,
                                                      unsigned long long* __restrict__ clock_sums) {
  const int first = (int)(blockIdx.x >> 8), rounds = (int)(gridDim.x >> 8);
  const int total = tab->total_tiles;
  for (int r = first;; r += rounds) {
    const int sidx = r * 8 + (int)(blockIdx.x & 7);
    if (sidx >= total) break;
    if (r != first) __syncthreads();  // every wave is done with the previous tile's LDS stages
    mxfp4_tile<PHASE>(bsrc, perm_src, tab, slot_base, slot_stride, code_off, scale_off, N, K, I, H, hout, yout,
                      clock_sums, sidx, (int)((blockIdx.x >> 3) & 31));
  }
}

// Per expert, a super-tile is GM token tiles x GN weight tiles (GM*GN <= 32
// block slots): GM = the smallest power of two covering its token tiles, at
// most 8; GN = the largest power of two dividing the weight tiles that fits
// beside it. Super-tiles per expert: ceil(m tiles / GM) x (n tiles / GN).
// Returns that count for a group of `rows` rows (0 for none) and sets
// shape = GM | GN << 8. Host planner and device planner use the same rule.
__host__ __device__ inline int supertiles_of(int rows, int N, int tile_tokens, int& shape) {
  const int NTB = N / 256;
  int gn_div = 1;
  while (gn_div < 16 && NTB % (gn_div * 2) == 0) gn_div *= 2;
  const int mtiles = (rows + tile_tokens - 1) / tile_tokens;
  int GM = 8;
  while (GM > 1 && GM / 2 >= mtiles) GM /= 2;
  const int GN = (32 / GM) < gn_div ? 32 / GM : gn_div;
  shape = GM | (GN << 8);
  return rows > 0 ? (mtiles + GM - 1) / GM * (NTB / GN) : 0;
}

// Fills item[i].w with GM | GN << 8 and tile_prefix; returns the total.
int plan_supertiles(int4* item, int n, int* tile_prefix, int N, int tile_tokens) {
  int tot = 0;
  for (int i = 0; i < n; ++i) {
    tile_prefix[i] = tot;
    int shape = 0;
    tot += supertiles_of(item[i].z, N, tile_tokens, shape);
    item[i].w = shape;
  }
  tile_prefix[n] = tot;
  return tot;
}

inline int supertile_blocks(int tot) { return (tot + 7) / 8 * 256; }  // 8 XCDs x 32 slots per round

// Up to 64 entries of both projections' tables per upload launch: the two
// share the items' slot and rows and differ in the super-tile shape (item.w)
// and the prefix sums.
struct TableChunk {
  int base, count, n, total[2];
  int prefix[2][64];
  int4 item[64];  // .w: the gate/up GEMM's GM | GN << 8
  int w2[64];     // the down GEMM's GM | GN << 8
};

__global__ __launch_bounds__(64) void table_upload(const TableChunk c, GemmTable* __restrict__ t1,
                                                   GemmTable* __restrict__ t2) {
  const int i = threadIdx.x;
  if (i < c.count) {
    const int4 it = c.item[i];
    t1->item[c.base + i] = it;
    t2->item[c.base + i] = make_int4(it.x, it.y, it.z, c.w2[i]);
    t1->tile_prefix[c.base + i] = c.prefix[0][i];
    t2->tile_prefix[c.base + i] = c.prefix[1][i];
  }
  if (i == 0 && c.base + c.count == c.n) {
    t1->tile_prefix[c.n] = c.total[0];
    t2->tile_prefix[c.n] = c.total[1];
  }
  if (i == 0 && c.base == 0) {
    t1->n = c.n;
    t1->total_tiles = c.total[0];
    t2->n = c.n;
    t2->total_tiles = c.total[1];
  }
}

// Plans both projections of the n items (gate/up N = 2I, down N = H; tiles
// of tile_tokens) and writes their tables; tot receives the super-tile counts.
hipError_t plan_and_upload(const int4* items, int n, int H, int I, int tile_tokens, GemmTable* t1, GemmTable* t2,
                           int (&tot)[2], hipStream_t s) {
  std::vector<int4> it1(items, items + n), it2(items, items + n);
  std::vector<int> pre1(n + 1), pre2(n + 1);
  tot[0] = plan_supertiles(it1.data(), n, pre1.data(), 2 * I, tile_tokens);
  tot[1] = plan_supertiles(it2.data(), n, pre2.data(), H, tile_tokens);
  TableChunk c;
  for (int base = 0; base < n; base += 64) {
    memset(&c, 0, sizeof c);
    c.base = base;
    c.count = n - base < 64 ? n - base : 64;
    c.n = n;
    c.total[0] = tot[0];
    c.total[1] = tot[1];
    for (int i = 0; i < c.count; ++i) {
      c.item[i] = it1[base + i];
      c.w2[i] = it2[base + i].w;
      c.prefix[0][i] = pre1[base + i];
      c.prefix[1][i] = pre2[base + i];
    }
    hipLaunchKernelGGL(table_upload, dim3(1), dim3(64), 0, s, c, t1, t2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Device planner of the grouped GEMM's work list: one block, thread e for
// expert e (E <= 1024). Expert e has counts[e] rows from offsets[e] of the
// grouped layout and its blob at slot slot_of[e] (slot_of NULL: slot e).
// Groups go to part 0 when they have more than `split` rows, to part 1 when
// they have 1..split rows; for each part and projection (N1 = gate/up rows,
// N2 = down rows) the items are written in ascending expert order with the
// super-tile prefix sums of supertiles_of, as the host planner writes them.
// A group that would reach past row `rows_max` or whose slot lies outside
// [0, n_slots) is left out (its rows are not computed).
__global__ __launch_bounds__(1024) void plan_tables_kernel(const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ slot_of, int E, int n_slots,
                                                           int rows_max, int N1, int N2, int split, int tt0, int tt1,
                                                           char* __restrict__ tables) {
  constexpr int NV = 6;  // member of part 0, part 1; super-tiles (part 0, N1), (0, N2), (1, N1), (1, N2)
  __shared__ int wave_tot[16][NV];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int rows = 0, begin = 0, slot = 0;
  if (e < E) {
    rows = counts[e];
    begin = offsets[e];
    slot = slot_of ? slot_of[e] : e;
    if (rows < 0 || begin < 0 || (long long)begin + rows > rows_max || slot < 0 || slot >= n_slots) rows = 0;
  }
  const int part = rows > split ? 0 : (rows > 0 ? 1 : -1);
  int shape[2][2] = {{0, 0}, {0, 0}};
  int v[NV] = {part == 0, part == 1, 0, 0, 0, 0};
  if (part >= 0) {
    const int tt = part == 0 ? tt0 : tt1;
    v[2 + 2 * part] = supertiles_of(rows, N1, tt, shape[part][0]);
    v[3 + 2 * part] = supertiles_of(rows, N2, tt, shape[part][1]);
  }
  int inc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int x = v[i];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    inc[i] = x;
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NV; ++i) wave_tot[wave][i] = inc[i];
  }
  __syncthreads();
  int ex[NV], tot[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int before = 0, all = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      if (w < wave) before += wave_tot[w][i];
      all += wave_tot[w][i];
    }
    ex[i] = before + inc[i] - v[i];
    tot[i] = all;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      GemmTable* t = reinterpret_cast<GemmTable*>(tables + (2 * p + ph) * kTableBytes);
      if (part == p) {
        t->item[ex[p]] = make_int4(slot, begin, rows, shape[p][ph]);
        t->tile_prefix[ex[p]] = ex[2 + 2 * p + ph];
      }
      if (e == 0) {
        t->n = tot[p];
        t->total_tiles = tot[2 + 2 * p + ph];
        t->tile_prefix[tot[p]] = tot[2 + 2 * p + ph];
      }
    }
  }
}

}  // namespace

bool gemm2_supported(int N, int K) { return N % 256 == 0 && K % 32 == 0; }

void set_clock_sums(unsigned long long* sums) { g_clock_sums = sums; }

// Both projections of every listed expert: groups of more than 256 rows with
// 256-token tiles (8 waves of 128 x 64), the others with 128-token tiles
// (8 waves of 64 x 64); one launch per tile size and projection, each with
// its whole work list in a device table.
hipError_t launch_ffn_prefill2(const void* x, const int32_t* perm_src, const int4* items, int n,
                               const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                               void* tables, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > kTableItems) return hipErrorInvalidValue;
  const BlobLayout L = blob_layout(1, H, I);
  std::vector<int4> part[2];  // [0] groups of more than 256 rows, [1] the rest
  for (int i = 0; i < n; ++i) part[items[i].z > 256 ? 0 : 1].push_back(items[i]);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* hb = static_cast<uint16_t*>(hbuf);
  GemmTable* tab[2][2];  // [part][projection]
  int tot[2][2] = {{0, 0}, {0, 0}};
  for (int p = 0; p < 2; ++p) {
    for (int ph = 0; ph < 2; ++ph)
      tab[p][ph] = reinterpret_cast<GemmTable*>(static_cast<char*>(tables) + (2 * p + ph) * kTableBytes);
    const int m = (int)part[p].size();
    if (m == 0) continue;
    hipError_t e = plan_and_upload(part[p].data(), m, H, I, p == 0 ? 256 : 128, tab[p][0], tab[p][1], tot[p], s);
    if (e != hipSuccess) return e;
  }
  if (tot[0][0] > 0)
    hipLaunchKernelGGL((gemm2_bf16<1, 16, const GemmTable*>), dim3(supertile_blocks(tot[0][0])), dim3(512), 0, s, xb,
                       perm_src, (const GemmTable*)tab[0][0], slot_base, slot_stride, L.p1, 2 * I, H, H, I, hb, y,
                       nullptr, g_clock_sums);
  if (tot[1][0] > 0)
    hipLaunchKernelGGL((gemm2_bf16<1, 8, const GemmTable*>), dim3(supertile_blocks(tot[1][0])), dim3(512), 0, s, xb,
                       perm_src, (const GemmTable*)tab[1][0], slot_base, slot_stride, L.p1, 2 * I, H, H, I, hb, y,
                       nullptr, g_clock_sums);
  if (tot[0][1] > 0)
    hipLaunchKernelGGL((gemm2_bf16<2, 16, const GemmTable*>), dim3(supertile_blocks(tot[0][1])), dim3(512), 0, s, hb,
                       perm_src, (const GemmTable*)tab[0][1], slot_base, slot_stride, L.p2, H, I, H, I, hb, y,
                       nullptr, g_clock_sums);
  if (tot[1][1] > 0)
    hipLaunchKernelGGL((gemm2_bf16<2, 8, const GemmTable*>), dim3(supertile_blocks(tot[1][1])), dim3(512), 0, s, hb,
                       perm_src, (const GemmTable*)tab[1][1], slot_base, slot_stride, L.p2, H, I, H, I, hb, y,
                       nullptr, g_clock_sums);
  return hipGetLastError();
}

bool prefill_mxfp4_supported(int H, int I) { return H % 256 == 0 && I % 128 == 0; }

// Both projections of every listed expert with MXFP4 weights: 128-token
// tiles, one launch per projection, the work list in a device table.
hipError_t launch_ffn_prefill_mxfp4(const void* x, const int32_t* perm_src, const int4* items, int n,
                                    const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                                    void* tables, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > kTableItems || !prefill_mxfp4_supported(H, I)) return hipErrorInvalidValue;
  const BlobLayout L = blob_layout(3, H, I);
  int tot[2] = {0, 0};
  GemmTable* tab[2];
  for (int ph = 0; ph < 2; ++ph) tab[ph] = reinterpret_cast<GemmTable*>(static_cast<char*>(tables) + ph * kTableBytes);
  hipError_t e = plan_and_upload(items, n, H, I, 128, tab[0], tab[1], tot, s);
  if (e != hipSuccess) return e;
  uint16_t* hb = static_cast<uint16_t*>(hbuf);
  if (tot[0] > 0)
    hipLaunchKernelGGL(gemm_mxfp4<1>, dim3(supertile_blocks(tot[0])), dim3(512), 0, s,
                       static_cast<const uint16_t*>(x), perm_src, (const GemmTable*)tab[0], slot_base, slot_stride,
                       L.p1, L.p1s, 2 * I, H, I, H, hb, y, g_clock_sums);
  if (tot[1] > 0)
    hipLaunchKernelGGL(gemm_mxfp4<2>, dim3(supertile_blocks(tot[1])), dim3(512), 0, s, hb, perm_src,
                       (const GemmTable*)tab[1], slot_base, slot_stride, L.p2, L.p2s, H, I, I, H, hb, y,
                       g_clock_sums);
  return hipGetLastError();
}

bool grouped_supported(int wfmt, int H, int I) {
  if (wfmt == 1) return gemm2_supported(2 * I, H) && gemm2_supported(H, I);
  if (wfmt == 3) return prefill_mxfp4_supported(H, I);
  return false;
}

// Both projections of every expert with rows, the work list planned on the
// device from counts and offsets (no host synchronisation): bf16 weights in
// the two tile sizes of launch_ffn_prefill2, MXFP4 weights in 128-token tiles.
// Each GEMM launch is a fixed number of rounds of 256 blocks whose blocks
// loop over the super-tiles the planner wrote.
hipError_t launch_ffn_grouped(int wfmt, const void* x, const int32_t* perm_src, const int32_t* counts,
                              const int32_t* offsets, const int32_t* slot_of, int E, int n_slots, int rows_max,
                              const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                              void* tables, hipStream_t s) {
  if (E < 1 || E > kTableItems || !grouped_supported(wfmt, H, I)) return hipErrorInvalidValue;
  const bool mx = wfmt == 3;
  char* tb = static_cast<char*>(tables);
  hipLaunchKernelGGL(plan_tables_kernel, dim3(1), dim3((E + 63) / 64 * 64), 0, s, counts, offsets, slot_of, E,
                     n_slots, rows_max, 2 * I, H, mx ? 0 : 256, mx ? 128 : 256, 128, tb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const GemmTable* tab[2][2];
  for (int p = 0; p < 2; ++p)
    for (int ph = 0; ph < 2; ++ph) tab[p][ph] = reinterpret_cast<const GemmTable*>(tb + (2 * p + ph) * kTableBytes);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* hb = static_cast<uint16_t*>(hbuf);
  const dim3 block(512);
  // Rounds of 256 blocks per launch. A block whose slot a super-tile leaves empty moves on to its next round,
  // so with a single round those blocks' CUs would idle: 32 / (fewest slots a super-tile can fill) rounds let
  // the blocks of empty slots exit and others take their CUs. Eight times that many keeps each block's list of
  // super-tiles short, so the dispatcher hands the next block to whichever CU frees first and the blocks of a
  // super-tile stay close to each other in K (one resident 16384-token Zipf layer: 5.24-5.50 ms with the
  // fewer, longer-lived blocks, 4.95-5.16 ms with these; results bit-identical).
  const auto grid = [](int N, int gm_min) {
    int GM = gm_min, shape = 0;
    supertiles_of(GM * 128, N, 128, shape);  // shape of the smallest super-tile a group of this part gets
    const int fill = (shape & 0xFF) * (shape >> 8);
    return dim3(256 * 8 * (fill >= 32 ? 1 : 32 / fill));
  };
  if (mx) {
    // split 0 puts every group with rows into part 0, planned with 128-token tiles
    const BlobLayout L = blob_layout(3, H, I);
    hipLaunchKernelGGL(gemm_mxfp4<1>, grid(2 * I, 1), block, 0, s, xb, perm_src, tab[0][0], slot_base, slot_stride,
                       L.p1, L.p1s, 2 * I, H, I, H, hb, y, g_clock_sums);
    hipLaunchKernelGGL(gemm_mxfp4<2>, grid(H, 1), block, 0, s, hb, perm_src, tab[0][1], slot_base, slot_stride, L.p2,
                       L.p2s, H, I, I, H, hb, y, g_clock_sums);
    return hipGetLastError();
  }
  // part 0 groups (more than 256 rows) have at least two 256-token tiles, part 1 groups one or two 128-token tiles
  const BlobLayout L = blob_layout(1, H, I);
  hipLaunchKernelGGL((gemm2_bf16<1, 16, const GemmTable*>), grid(2 * I, 2), block, 0, s, xb, perm_src, tab[0][0],
                     slot_base, slot_stride, L.p1, 2 * I, H, H, I, hb, y, nullptr, g_clock_sums);
  hipLaunchKernelGGL((gemm2_bf16<1, 8, const GemmTable*>), grid(2 * I, 1), block, 0, s, xb, perm_src, tab[1][0],
                     slot_base, slot_stride, L.p1, 2 * I, H, H, I, hb, y, nullptr, g_clock_sums);
  hipLaunchKernelGGL((gemm2_bf16<2, 16, const GemmTable*>), grid(H, 2), block, 0, s, hb, perm_src, tab[0][1],
                     slot_base, slot_stride, L.p2, H, I, H, I, hb, y, nullptr, g_clock_sums);
  hipLaunchKernelGGL((gemm2_bf16<2, 8, const GemmTable*>), grid(H, 1), block, 0, s, hb, perm_src, tab[1][1],
                     slot_base, slot_stride, L.p2, H, I, H, I, hb, y, nullptr, g_clock_sums);
  return hipGetLastError();
}

// Router logits on matrix cores, split over K into `nsplit` slabs of partial
// sums: partial[(z * T + t) * E + e] over the z-th H / nsplit columns (no
// bias; the top-k kernel adds the slabs in order, then the bias).
int router_gemm2_splits(int T, int H, int E) {
  const int tiles = (T + 127) / 128 * (E / 256);
  int S = 1;
  while (S < 16 && tiles * S < 256 && (H / 32) % (2 * S) == 0 && H / 32 / (2 * S) >= 4) S *= 2;
  return S;
}

hipError_t launch_router_gemm2(const void* x, const void* wrt, int T, int H, int E, float* partial, int nsplit,
                               hipStream_t s) {
  if (nsplit < 1 || nsplit > kMaxItems || (H / 32) % nsplit != 0) return hipErrorInvalidValue;
  WorkArgs wa;
  memset(&wa, 0, sizeof wa);
  wa.n = nsplit;
  for (int z = 0; z < nsplit; ++z) wa.item[z] = make_int4(z, 0, T, 0);
  wa.total_tiles = plan_supertiles(wa.item, nsplit, wa.tile_prefix, E, 128);
  if (wa.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm2_bf16<0, 8, WorkArgs>), dim3(supertile_blocks(wa.total_tiles)), dim3(512), 0, s,
                     static_cast<const uint16_t*>(x), nullptr, wa, static_cast<const char*>(wrt), 0, 0, E, H / nsplit,
                     H, 0, nullptr, partial, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
