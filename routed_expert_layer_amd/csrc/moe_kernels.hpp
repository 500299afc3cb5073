// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace moe {

// ---------------------------------------------------------------------------
// Expert blob layouts.
//
// bf16 (MOE_W_BF16): two weight matrices stored as matrix-core fragments.
//   P1 = the gate and up projections, N1 = 2I output rows, K1 = H.
//   P2 = the down projection,        N2 = H  output rows, K2 = I.
//   A matrix with N rows and K columns is cut into N/16 row tiles; a row tile
//   is K/32 fragments of 1 KiB, in K order; fragment byte 16*l..16*l+15
//   holds row (l % 16) of the tile, columns 32c + 8(l/16) .. +7 (8 bf16).
//   This is the A-operand register layout of v_mfma_f32_16x16x32_bf16, so
//   one wave streams a fragment with a single coalesced 1 KiB load.
//   P1 row r of tile t (q = (r%16)/4, s = r%4) is column i = 8t + 2q + s/2
//   of W1 (s even) or W3 (s odd): the accumulator lane that ends up with
//   rows 4q..4q+3 holds gate and up values of two consecutive i.
//   P2 row n is column n of W2.
// int4 (MOE_W_INT4): the same row order. A row tile is K/128 blocks of 1 KiB;
//   block g, byte 16*l..16*l+15 = four 32-bit words, word j holding the codes
//   of row (l%16), columns 128g + 32j + 8(l/16) + 0..7 as nibbles
//   (nibble p, bits 4p..4p+3): code(k0),code(k2),code(k4),code(k6),
//   code(k1),code(k3),code(k5),code(k7); nibble = q + 8.
//   Scales: per row tile and block, the 16 rows' fp16 scales (32 B).
//   Sections: [P1 codes][P1 scales][P2 codes][P2 scales], 256-B aligned.
// MXFP4 (MOE_W_MXFP4): the same row order. A row tile is K/128 blocks of
//   1 KiB of FP4 (E2M1) codes; block g, byte 16*l..16*l+15 = four 32-bit
//   words, word j holding row (l%16), columns 128g + 32j + 8(l/16) + 0..7
//   as nibbles in column order (nibble p = bits 4p..4p+3).
//   Scales: per row tile and block, 64 bytes of E8M0 scales, byte 4r + j =
//   scale of row r, columns 128g + 32j .. +31 (one scale per 32 of K).
//   Sections: [P1 codes][P1 scales][P2 codes][P2 scales], 256-B aligned.
// fp32 (MOE_W_F32): W1 [H,I], W3 [H,I], W2 [I,H] row-major, concatenated.
// ---------------------------------------------------------------------------
struct BlobLayout {
  size_t p1, p1s, p2, p2s, bytes;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline BlobLayout blob_layout(int wfmt, int H, int I) {
  BlobLayout b{};
  const size_t HI = (size_t)H * I;
  if (wfmt == 0) {  // fp32
    b.p1 = 0; b.p2 = 2 * HI * 4; b.bytes = 3 * HI * 4;
  } else if (wfmt == 1) {  // bf16
    b.p1 = 0; b.p2 = 2 * HI * 2; b.bytes = 3 * HI * 2;
  } else if (wfmt == 3) {  // MXFP4
    b.p1 = 0;
    b.p1s = align_up(HI, 256);                                   // 2HI codes * 0.5 B
    b.p2 = align_up(b.p1s + (size_t)(2 * I / 16) * (H / 128) * 64, 256);
    b.p2s = align_up(b.p2 + HI / 2, 256);
    b.bytes = align_up(b.p2s + (size_t)(H / 16) * (I / 128) * 64, 256);
  } else {  // int4
    b.p1 = 0;
    b.p1s = align_up(b.p1 + HI, 256);                       // 2HI codes * 0.5 B
    b.p2 = align_up(b.p1s + (size_t)(2 * I / 16) * (H / 128) * 32, 256);
    b.p2s = align_up(b.p2 + HI / 2, 256);
    b.bytes = align_up(b.p2s + (size_t)(H / 16) * (I / 128) * 32, 256);
  }
  return b;
}

// P1 row r (0..2I-1) -> (matrix 0 = W1 / 1 = W3, column i).
__host__ __device__ inline void p1_row_source(int r, int& mat, int& i) {
  const int t = r >> 4, rr = r & 15, q = rr >> 2, s = rr & 3;
  i = 8 * t + 2 * q + (s >> 1);
  mat = s & 1;
}

// Work items passed by value in the kernel arguments.
constexpr int kMaxItems = 64;
struct WorkArgs {
  int n;
  int total_tiles;
  int tile_prefix[kMaxItems + 1];  // prefix sums of per-item tile counts (prefill GEMM)
  int4 item[kMaxItems];            // {slot, row_begin, rows, expert}
};

// Work list of one prefill GEMM launch, in device memory (written by a small
// upload kernel), so one launch covers every expert of a layer.
constexpr int kTableItems = 1024;
struct GemmTable {
  int n;
  int total_tiles;
  int pad_[2];
  int tile_prefix[kTableItems + 1];  // super-tile prefix sums
  int4 item[kTableItems];            // {slot, row_begin, rows, GM | GN << 8}
};
constexpr size_t kTableBytes = (sizeof(GemmTable) + 255) / 256 * 256;

// ---------------------------------------------------------------------------
// Launchers (return hipError_t of the launch).
// ---------------------------------------------------------------------------
size_t route_workspace_bytes(int T, int H, int E, int k);
// The host-driven decoder's copy of the cache's slot table on the GPU
// (slot_of[key], -1: not resident): updates to it (distinct keys), and the
// list of a layer-step's experts it shows as resident, as FFN work items
// {slot, first row, rows, expert} in ascending expert order.
constexpr int kSlotUpdatesMax = 64;
struct SlotUpdates {
  int n;
  int32_t key[kSlotUpdatesMax], slot[kSlotUpdatesMax];
};
// Device-resident cache control (kernels_devctl.hip). All pointers are device
// memory owned by a device-controlled decoder.
struct DevCache {
  int32_t* slot_of;   // [L*E] key -> slot, -1 if not resident
  int32_t* slot_key;  // [S] slot -> key, -1 if free
  uint64_t* stamp;    // [S] last use (clock value) of each occupied slot
  uint64_t* ctl;      // [0] clock, [1] hits, [2] misses, [3] resolve calls, [4] trace records
  int S;
  int4* work;         // [max items] {slot, row_begin, rows, expert}: hits, then misses
  int4* miss;         // [max items] {expert, slot, victim key or -1, key}
  int32_t* n;         // [0] work items, [1] misses, [2] hits (of the last resolve)
  int32_t* trace;     // [trace_cap][7] records as moe_trace_t
  int64_t trace_cap;
};
// A device-controlled decoder's resolve of one layer-step, run by the routing
// launch itself on the decode-size path.
struct DevStep {
  DevCache c;  // c.slot_of == nullptr: none
  int layer;
};
struct ResidentList {
  int32_t* slot_of;     // nullptr: no list
  int layer;
  int32_t* n_out;       // [2]: items listed, experts with tokens
  int4* items;          // [E]
  SlotUpdates updates;  // applied to slot_of before the list is made
};
hipError_t launch_route(const void* x, bool bf16, const void* Wr, const float* bias, int T, int H, int E, int k,
                        int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts, int32_t* offsets,
                        int32_t* perm_src, int32_t* perm_pos, void* ws, hipStream_t s,
                        // optional host-mapped copy of counts: for batches of at most 16 tokens and 512 experts
                        // (route_small_path) each word is (mirror_seq << 16) | count, mirror_seq in 1..65535;
                        // for other batches plain counts
                        int32_t* counts_mirror = nullptr, int32_t mirror_seq = 0,
                        // optional, decode-size path only: the resident experts' work list (see ResidentList)
                        const ResidentList* resident = nullptr,
                        // optional, decode-size path only: the device-resident cache's resolve of this layer-step
                        // (as launch_dev_resolve), run at the end of the last routing kernel
                        const DevStep* dev = nullptr);
// Whether launch_route takes the decode-size path (and tags its counts mirror).
bool route_small_path(int T, int E);

hipError_t launch_pack(int wfmt, int H, int I, const void* W1, const void* W3, const void* W2,
                       const void* s1, const void* s3, const void* s2, void* blob, hipStream_t s);

// Debug: n bytes at p set to 0xFF on stream s.
hipError_t launch_poison(void* p, size_t n, hipStream_t s);

hipError_t launch_combine(const float* y_perm, const int32_t* perm_pos, const float* w, int T, int k, int H,
                          void* out, bool out_bf16, hipStream_t s);

// FFN: decode (matrix-vector) kernels for groups of <= 16*? rows, prefill GEMM otherwise.
hipError_t launch_ffn_decode(int wfmt, const void* x, const int32_t* perm_src, const WorkArgs& wa,
                             const char* slot_base, size_t slot_stride, int H, int I,
                             void* hbuf, float* y, hipStream_t s);
// The same kernels with the work list in device memory: *n_items items at
// `items` (device), at most max_items of them with at most max_rows rows
// each; launch shapes depend only on max_items and max_rows. With `pool`
// set (not for fp32), items from *n_hit on are misses whose blob is read
// from pool + expert * pool_stride and written through into their slot;
// without it every item is resident and the kernels have no write-through
// path.
hipError_t launch_ffn_decode_dev(int wfmt, const void* x, const int32_t* perm_src, const int32_t* n_items,
                                 const int4* items, int max_items, int max_rows, const char* slot_base,
                                 size_t slot_stride, int H, int I, void* hbuf, float* y, hipStream_t s,
                                 const int32_t* n_hit = nullptr, const char* pool = nullptr,
                                 size_t pool_stride = 0);
// Both projections of the quantised decode FFN of experts listed in device
// memory, as launch_ffn_decode_dev (with or without `pool`), in one launch:
// the down-projection blocks wait for their expert's gate/up blocks through
// `flags` (device, ffn_fused_flags(max_items, I) 64-bit words, zero before
// the first call, owned by one caller whose calls are stream-ordered). Each
// call needs a flag value no earlier call used: a nonzero `seq`, or with
// seq_dev set, one above the value at seq_dev when the call runs (a counter
// the caller's earlier work advances by one per call). ffn_fused_ok tells
// whether a format and shape take this path.
bool ffn_fused_ok(int wfmt, int H, int I);
size_t ffn_fused_flags(int max_items, int I);
hipError_t launch_ffn_decode_fused(int wfmt, const void* x, const int32_t* perm_src, const int32_t* n_items,
                                   const int4* items, int max_items, const char* slot_base, size_t slot_stride, int H,
                                   int I, void* hbuf, float* y, uint64_t* flags, uint64_t seq, hipStream_t s,
                                   const uint64_t* seq_dev = nullptr, const int32_t* n_hit = nullptr,
                                   const char* pool = nullptr, size_t pool_stride = 0);
// The bf16 decode FFN of the experts listed in device memory (at most
// kFuseItems items, *n_items of them; with `pool`, items from *n_hit on are
// misses read from the pool and written through into their slots, as for
// launch_ffn_decode_dev) with the step's weighted combine in the down
// projection: y_perm gets every listed item's rows, and when
// *n_active == *n_items (no expert of the step is left out) `out` [T, H]
// (fp32, or bf16 with out_bf16) gets the combine's result, summed in the
// combine kernel's order; otherwise `out` is left alone. ffn_combine_ok
// tells whether a shape can take this path.
constexpr int kFuseItems = 8;
bool ffn_combine_ok(int wfmt, int H, int I, int max_items, int T, int k);
hipError_t launch_ffn_decode_combine(const void* x, const int32_t* perm_src, const int32_t* n_items, const int4* items,
                                     int max_items, int T, const char* slot_base, size_t slot_stride, int H, int I,
                                     void* hbuf, float* y_perm, const int32_t* n_active, const int32_t* perm_pos,
                                     const float* topk_w, int k, void* out, bool out_bf16, hipStream_t s,
                                     const int32_t* n_hit = nullptr, const char* pool = nullptr,
                                     size_t pool_stride = 0);
// 128 x 128-tile fallback GEMM for shapes the large-tile GEMM does not take.
hipError_t launch_ffn_prefill(const void* x, const int32_t* perm_src, WorkArgs& wa, const char* slot_base,
                              size_t slot_stride, int H, int I, void* hbuf, float* y, hipStream_t s);
bool prefill_supported(int wfmt, int H, int I);
// Matrix-core router for long batches: Wr [H, E] bf16 is first rearranged into
// fragment order (rows = experts, K = H) in the workspace, then
// logits[t, e] = x[t, :] . Wr[:, e] + bias[e] (fp32) by the GEMM kernel.
hipError_t launch_pack_fragments(const void* W, int K, int N, void* dst, hipStream_t s);
// Writes `nsplit` slabs of partial logits (no bias): partial[(z*T + t)*E + e].
// router_gemm_splits gives the slab count the launcher will use.
int router_gemm_splits(int T, int H, int E);
hipError_t launch_router_gemm(const void* x, const void* wrt, int T, int H, int E, float* partial, int nsplit,
                              hipStream_t s);
// Large-tile GEMM (256 weight rows per block) used when N % 256 == 0.
bool gemm2_supported(int N, int K);
// Clock diagnostic: while `sums` (device, two uint64) is set, every block of
// the prefill expert GEMMs adds the shader-clock cycles and 100 MHz real-time
// ticks it spent up to its epilogue to sums[0] and sums[1]; nullptr turns it
// off. Process-wide, read at each launch.
void set_clock_sums(unsigned long long* sums);
// Both projections of n work items {slot, row_begin, rows, expert} (host
// array, rows > 0, n <= kTableItems) with four GemmTables at `tables`
// (4 * kTableBytes of device memory, stream-ordered reuse).
hipError_t launch_ffn_prefill2(const void* x, const int32_t* perm_src, const int4* items, int n,
                               const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                               void* tables, hipStream_t s);
// The same with MXFP4 weights (128-token tiles; two GemmTables at `tables`).
bool prefill_mxfp4_supported(int H, int I);
hipError_t launch_ffn_prefill_mxfp4(const void* x, const int32_t* perm_src, const int4* items, int n,
                                    const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                                    void* tables, hipStream_t s);
// Shapes the device-planned grouped GEMM takes: bf16 with 2I and H multiples
// of 256 (I a multiple of 32), MXFP4 as prefill_mxfp4_supported.
bool grouped_supported(int wfmt, int H, int I);
// Both projections of every expert e of 0..E-1 with counts[e] > 0 rows at
// offsets[e] of the grouped layout (device arrays, e.g. moe_route's), blob at
// slot slot_of[e] (device, NULL: e) of slot_base; the work list is planned on
// the device into the four GemmTables at `tables`, so nothing waits for the
// GPU. Groups reaching past rows_max or with a slot outside [0, n_slots) are
// skipped.
hipError_t launch_ffn_grouped(int wfmt, const void* x, const int32_t* perm_src, const int32_t* counts,
                              const int32_t* offsets, const int32_t* slot_of, int E, int n_slots, int rows_max,
                              const char* slot_base, size_t slot_stride, int H, int I, void* hbuf, float* y,
                              void* tables, hipStream_t s);
int router_gemm2_splits(int T, int H, int E);
hipError_t launch_router_gemm2(const void* x, const void* wrt, int T, int H, int E, float* partial, int nsplit,
                               hipStream_t s);

// One layer-step of the policy on the device (one workgroup; E <= 1024).
hipError_t launch_slot_updates(int32_t* slot_of, const SlotUpdates& u, hipStream_t s);

hipError_t launch_dev_resolve(const int32_t* counts, const int32_t* offsets, int E, int layer, const DevCache& c,
                              hipStream_t s);
// Copies the last resolve's misses from `pool` (device-visible address of the
// layer's pinned pool) into their slots; fixed grid, exits when there are none.
hipError_t launch_dev_fill(const DevCache& c, const void* pool, size_t blob_stride, size_t blob_bytes,
                           void* slot_base, size_t slot_stride, hipStream_t s);

// Host: reads one byte per page of a pool region on the CPU thread pool.
void cpu_touch_pages(const void* p, size_t bytes);

// Sets the calling thread's moe_last_error() message; returns `code`.
int set_error(int code, const char* fmt, ...);

constexpr int kGemmBM = 128;  // tokens per GEMM tile
constexpr int kGemmBN = 128;  // output rows per GEMM tile

}  // namespace moe
