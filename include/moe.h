/*
 * moe.h -- C ABI of the routed expert layer for AMD Instinct MI355X (gfx950).
 *
 * The layer: a router picks k experts per token, the selected (layer, expert)
 * pairs are resolved against a shared LRU expert cache held in GPU memory,
 * missing experts are copied from a pinned host-resident pool, tokens are
 * grouped by expert, every expert runs a SwiGLU FFN, and the expert outputs
 * are combined with the routing weights.
 *
 * Sources. Page "FreeToken-rtx-4090" (freetoken.wiki), sections "Overview",
 * "How the MoE Memory Hierarchy Works" and its component table; page
 * "FreeToken-benchmark", section "How FreeToken Serves Large MoE Models". The
 * pages describe the system (host pool, elastic GPU cache keyed by
 * layer-and-expert, shared LRU in decode, full-layer double buffering in
 * prefill, fills over a measured PCIe path) but not the arithmetic of the
 * layer; the arithmetic each call performs is stated with the call.
 *
 * Conventions (all calls):
 *  - Return value: MOE_OK (0) or a negative MOE_E* code; moe_last_error()
 *    then holds a message for the calling thread. No call aborts the process
 *    and no C++ exception crosses this interface.
 *  - "device" pointers are GPU memory (hipMalloc or a torch CUDA tensor),
 *    "host" pointers are CPU memory. The caller owns every buffer it passes;
 *    the library never frees caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls taking a stream only enqueue work; they return before it runs.
 *  - Matrices are row-major. bf16 is the 16-bit brain float (upper half of an
 *    IEEE fp32), fp16 is IEEE binary16.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* null or inconsistent argument */
  MOE_ECAPACITY = -2,  /* cache has no slots, or a request exceeds its capacity */
  MOE_EHIP = -3,       /* a HIP runtime call failed; its text is in moe_last_error() */
  MOE_ENOMEM = -4,     /* host or device allocation failed */
  MOE_ESTATE = -5      /* object used in a state that does not allow the call */
};

/* Activation / router element types. */
enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 };

/* Expert weight formats (the layout of one expert blob, see moe_pack_expert). */
enum { MOE_W_F32 = 0, MOE_W_BF16 = 1, MOE_W_INT4 = 2, MOE_W_MXFP4 = 3 };

/* FFN kernel choice for moe_ffn. */
enum { MOE_FFN_AUTO = 0, MOE_FFN_DECODE = 1, MOE_FFN_PREFILL = 2 };

/* Message for the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Interface version (increments on any incompatible change). */
int moe_abi_version(void);

/* ------------------------------------------------------------------------ *
 * Routing: router logits, top-k, combine weights and grouping by expert.
 *
 * Page "FreeToken-rtx-4090", section "How the MoE Memory Hierarchy Works":
 * each token activates a small subset of a layer's routed experts (six of
 * 256 in the model described). The pages do not define the gate; this call
 * computes the standard linear gate with softmax weights:
 *   l[t,e]   = sum_h x[t,h] * Wr[h,e] + bias[e]       (fp32 accumulation)
 *   S_t      = the k largest l[t,.], largest first; equal values go to the
 *              lower expert index; -0 equals +0
 *   w[t,j]   = exp(l[t,S_t[j]] - l[t,S_t[0]]) / sum_j' exp(l[t,S_t[j']] - l[t,S_t[0]])
 *   counts[e]   = number of (t, j) with S_t[j] = e
 *   offsets[e]  = sum_{e' < e} counts[e'],  offsets[E] = T*k
 *   perm_pos[t,j] = offsets[e] + #{t' < t : e in S_t'}   (e = S_t[j])
 *   perm_src[perm_pos[t,j]] = t
 * i.e. rows are grouped by ascending expert and, inside a group, ascending
 * token.
 *
 * x        device [T, H], element type `dtype` (MOE_DT_F32 or MOE_DT_BF16)
 * Wr       device [H, E], same element type as x
 * bias     device [E] fp32, or NULL for no bias
 * topk_idx device out int32 [T, k]      topk_w device out fp32 [T, k]
 * logits   device out fp32 [T, E] or NULL
 * counts   device out int32 [E]         offsets device out int32 [E+1]
 * perm_src device out int32 [T*k]       perm_pos device out int32 [T, k]
 * workspace device scratch of at least moe_route_workspace_size(T,H,E,k) bytes
 * Limits: 1 <= k <= min(E, 16), 1 <= E <= 1024, H % 8 == 0, T >= 0 (T = 0 is a
 * no-op that still writes counts = offsets = 0).
 * Errors: MOE_EINVAL for null required pointers or limits violated,
 * MOE_EHIP if a launch fails.
 * ------------------------------------------------------------------------ */
size_t moe_route_workspace_size(int T, int H, int E, int k);
int moe_route(const void* x, int dtype, const void* Wr, const float* bias,
              int T, int H, int E, int k,
              int32_t* topk_idx, float* topk_w, float* logits,
              int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* perm_pos,
              void* workspace, size_t ws_bytes, void* stream);

/* moe_route_noalloc: moe_route without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The routing kernels' scratch is a
 * device array of MOE_ROUTE_NOALLOC_MAX_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call allocates nothing and
 * enqueues only kernels. Arguments, results and errors as moe_route, plus
 * MOE_ECAPACITY when moe_route_workspace_size(T, H, E, k) exceeds
 * MOE_ROUTE_NOALLOC_MAX_BYTES (64 MiB: every batch up to 16384 tokens at H 4096,
 * E 256 fits; 16384 tokens at E 1024 do not).
 * All calls on one GPU share that scratch: calls that overlap on one GPU
 * (different streams, or different host threads) race and must be ordered by
 * the caller. */
#define MOE_ROUTE_NOALLOC_MAX_BYTES (64u << 20)
int moe_route_noalloc(const void* x, int dtype, const void* Wr, const float* bias,
                      int T, int H, int E, int k,
                      int32_t* topk_idx, float* topk_w, float* logits,
                      int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* perm_pos,
                      void* stream);

/* ------------------------------------------------------------------------ *
 * Expert blobs and the host pool.
 *
 * Page "FreeToken-rtx-4090": the complete expert pool lives in host memory
 * and is the source of truth ("Overview"; "How the MoE Memory Hierarchy
 * Works"), a cache entry is one complete layer-and-expert unit, and startup
 * loads weights straight into their final host layout (the phase table, row
 * "Startup"). Here one expert is one contiguous blob in the kernels' own
 * layout, so a cache fill is a single host-to-device copy.
 *
 * Canonical expert: W1, W3 [H, I] and W2 [I, H]; the expert computes
 *   y = (silu(x W1) * (x W3)) W2,  silu(z) = z / (1 + exp(-z)).
 * For MOE_W_INT4 the weights are q * s with int8 codes q in [-7, 7] of the
 * same shapes and fp16 scales s1, s3 [H/128, I], s2 [I/128, H]: one scale per
 * 128 consecutive rows (the reduction dimension K) and output column.
 * For MOE_W_MXFP4 (page "FreeToken-benchmark", model table: the routed
 * experts of DeepSeek-V4-Flash are deployed in MXFP4; the format is the OCP
 * Microscaling FP4 one) the weights are E2M1(c) * 2^(s - 127) with uint8 codes
 * c in 0..15 (bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa) of
 * the same shapes and uint8 E8M0 scales s1, s3 [H/32, I], s2 [I/32, H]: one
 * scale per 32 consecutive rows of K and output column. Supported scale bytes:
 * 1..254 with every dequantised weight a normal bf16 value (the kernels form
 * each weight exactly in bf16); activations stay bf16.
 *
 * moe_expert_bytes: size of one blob. Requirements: H and I multiples of 32
 * (bf16), of 128 (int4, MXFP4), I a multiple of 8; any H, I >= 1 for fp32.
 * moe_pack_expert: writes one blob from canonical device arrays, on `stream`.
 *   MOE_W_F32:  W1, W3, W2 fp32 device;  s1, s3, s2 ignored (NULL)
 *   MOE_W_BF16: W1, W3, W2 bf16 device;  s* ignored
 *   MOE_W_INT4: W1, W3, W2 are int8 codes (device), s1, s3, s2 fp16 device
 *   MOE_W_MXFP4: W1, W3, W2 are uint8 FP4 codes (device), s1, s3, s2 uint8
 *               E8M0 scales (device)
 *   blob: device out, moe_expert_bytes() bytes; the caller may then copy it
 *   into a pool or a cache slot.
 * moe_pool_alloc: page-locked host memory (hipHostMalloc) for the pool;
 *   returns NULL and sets *status on failure. Free with moe_pool_free. Every
 *   page is read once by the host threads before returning, so that CPU
 *   execution from the pool (moe_cpu_ffn) does not pay a first-touch cost.
 * ------------------------------------------------------------------------ */
size_t moe_expert_bytes(int wfmt, int H, int I);
int moe_pack_expert(int wfmt, int H, int I, const void* W1, const void* W3, const void* W2,
                    const void* s1, const void* s3, const void* s2, void* blob, void* stream);
void* moe_pool_alloc(size_t bytes, int* status);
int moe_pool_free(void* pool);

/* ------------------------------------------------------------------------ *
 * Shared LRU expert cache (host policy).
 *
 * Page "FreeToken-rtx-4090", section "How the MoE Memory Hierarchy Works": a
 * cache entry is a logical layer-and-expert pair, and decode keeps recently
 * selected experts in one LRU cache shared across layers and tokens that
 * changes with the routing; page "FreeToken-benchmark", section "How
 * FreeToken Serves Large MoE Models", the decode paragraph. Key = layer*E +
 * expert; the cache has S slots of equal size in GPU memory.
 *
 * cache_resolve runs one layer-step on the host:
 *   W  = the given experts (ascending, unique) as keys layer*E + e
 *   hits = W keys resident at entry, misses = the others
 *   access order = hits ascending, then misses ascending; each access is
 *   least-recently-used bookkeeping; a miss takes the lowest free slot, else
 *   the slot of the least recently used entry (the victim, which is evicted)
 *   the accesses form waves of at most S consecutive entries: all entries of
 *   a wave are resident together; run a wave's FFN before filling the next.
 * Outputs (host arrays of capacity n): work_e[i], work_slot[i], work_wave[i]
 * in access order; misses[0..*n_miss) in access order; *n_waves.
 * Every access is appended to the cache's trace (moe_cache_trace).
 *
 * moe_cache_set_split (page "FreeToken-rtx-4090", component table rows "CPU"
 * and "PCIe link", section "Adaptive Misses"): misses are divided between
 * GPU fills and CPU execution from measured rates (any common unit, e.g. MB/s
 * of PCIe fills and of the host expert kernel). Of all misses since the call,
 * floor(rate_gpu * count / (rate_gpu + rate_cpu)) go to the GPU (carried
 * remainder); within a layer-step the lowest keys go first. The others are
 * returned by cache_resolve after the GPU accesses with work_slot = -1 and
 * work_wave = -1 (run them with moe_cpu_ffn from the pool), are not in
 * misses[], are not cached and leave the recency order alone; their trace
 * records have slot = victim = wave = -1. rate_cpu = 0 (the default) fills
 * every miss. Errors: MOE_EINVAL (negative rates, zero sum, null).
 * Errors: MOE_EINVAL (null, layer or expert out of range, experts not
 * ascending or not unique), MOE_ECAPACITY (S == 0 at create).
 *
 * moe_cache_invalidate: drop a key (e.g. after a failed fill) so that it is
 * not left half-resident; its slot becomes free. MOE_EINVAL if not resident.
 *
 * moe_cache_resize (page "FreeToken-rtx-4090", runtime layer table, row "GPU
 * memory": cache capacity can change during runtime; page
 * "FreeToken-benchmark", section "Elastic Cache": capacity is rebuilt at safe
 * points without reloading the host pool): at a point where no layer-step is
 * in flight, the cache gets S_new slots. The min(S_new, resident) most
 * recently used entries are kept with their recency order, the others are
 * evicted (no trace records); a kept entry in a slot below S_new keeps it, the
 * kept entries at or above S_new move, in ascending old slot, to the lowest
 * free slots below S_new. moves[0..*n_moves) lists them (key, old slot, new
 * slot): copy each blob before the slots are used again. Growing moves
 * nothing. Errors: ECAPACITY (S_new < 1), EINVAL (null, more moves than
 * max_moves; the cache is then unchanged). moe_cache_capacity: current S.
 * moe_cache_slot_of: *slot = slot of key or -1.
 * A handle must not be used from two threads at once.
 * ------------------------------------------------------------------------ */
typedef struct moe_cache moe_cache_t;
typedef struct { int32_t key, slot, victim, wave; } moe_miss_t;
typedef struct { int32_t key, from_slot, to_slot; } moe_move_t;
typedef struct { int32_t step, layer, key, hit, slot, victim, wave; } moe_trace_t;

moe_cache_t* moe_cache_create(int L, int E, int S, int* status);
int moe_cache_destroy(moe_cache_t* cache);
int cache_resolve(moe_cache_t* cache, int step, int layer, const int32_t* experts, int n,
                  int32_t* work_e, int32_t* work_slot, int32_t* work_wave,
                  moe_miss_t* misses, int* n_miss, int* n_waves);
int moe_cache_set_split(moe_cache_t* cache, int rate_gpu, int rate_cpu);
int moe_cache_trace(const moe_cache_t* cache, moe_trace_t* out, int64_t max_records, int64_t* n_records);
int moe_cache_clear_trace(moe_cache_t* cache);
int moe_cache_invalidate(moe_cache_t* cache, int key);
int moe_cache_slot_of(const moe_cache_t* cache, int key, int* slot);
int moe_cache_stats(const moe_cache_t* cache, int64_t* hits, int64_t* misses);
int moe_cache_resize(moe_cache_t* cache, int S_new, moe_move_t* moves, int max_moves, int* n_moves);
int moe_cache_capacity(const moe_cache_t* cache);

/* ------------------------------------------------------------------------ *
 * Miss fills over the host link.
 *
 * Page "FreeToken-rtx-4090", component table row "PCIe link" (only the misses
 * chosen for GPU execution move) and the paragraph after it (a missing expert
 * can be copied into the cache and executed on the GPU).
 *
 * cache_fill_async: for each miss, copies blob `key` of the pool
 * (layer_pool[key / E] + (key % E)*blob_stride, blob_bytes bytes; pinned host
 * memory; layer_pool holds the L per-layer base addresses, which may repeat
 * when layers share weights) to slot
 * `slot` (slot_base + slot*slot_stride; device). Ordering: the copies start
 * only after all work enqueued on compute_stream before this call (which
 * includes every earlier reader of a victim slot), run on fill_stream, and
 * work enqueued on compute_stream after this call waits for them.
 * fill_stream may equal compute_stream. Uses the cache's own events.
 * Errors: MOE_EINVAL (null, key or slot out of range, no pool address for a
 * layer), MOE_EHIP (copy or event failure). On any error no key of the batch
 * is left mapped to a slot its copy did not reach (page "FreeToken-rtx-4090",
 * component table, row "PCIe link": a miss moves as one complete expert): the
 * failed miss and every later one are dropped from the cache as by
 * moe_cache_invalidate (their slots become free); copies issued before the
 * failure keep their keys, and later compute-stream work is still ordered
 * after them (if the ordering itself fails, the whole batch is dropped).
 * Debug: with MOE_DEBUG_POISON_FILLS=1 in the environment when the cache is
 * created, every fill first sets its slot's blob_bytes to 0xFF (NaN in bf16,
 * fp32 and in the int4 and MXFP4 scales), so a read not ordered after the
 * copy, or a copy overwriting a slot still being read, shows as non-finite
 * output.
 * ------------------------------------------------------------------------ */
int cache_fill_async(moe_cache_t* cache, const moe_miss_t* misses, int n,
                     const void* const* layer_pool, size_t blob_stride, size_t blob_bytes,
                     void* slot_base, size_t slot_stride,
                     void* fill_stream, void* compute_stream);

/* ------------------------------------------------------------------------ *
 * Grouped expert FFN.
 *
 * Page "FreeToken-rtx-4090", section "How the MoE Memory Hierarchy Works": an
 * expert is one complete layer-and-expert unit, executed through the same
 * logical mapping wherever it is resident, and the GPU executes the experts
 * held in its cache (the paragraph after the component table: a missing
 * expert is either filled into the cache and run on the GPU or run on the
 * CPU). The pages do not write the expert's arithmetic; this call computes a
 * SwiGLU expert (gate on x W1, up on x W3, down W2), the grouped form the
 * layer is specified with.
 *
 * Runs each listed expert on its group of rows:
 *   for row r in [row_begin, row_begin + rows) of item i (expert blob at
 *   slot_base + slot*slot_stride):
 *     xr = x[perm_src[r], :]
 *     y_perm[r, :] = (silu(xr W1) * (xr W3)) W2          (fp32 out)
 * Accumulation is fp32. In the matrix-core kernels (bf16, int4 and MXFP4
 * weights) x enters as given (bf16) and the SwiGLU product is rounded to bf16
 * before the W2 product. An int4 code q enters the bf16 products exactly as
 * 1 + (q + 8)/16; a 128-row block's sum over q is recovered in fp32 as
 * 16 t - 24 u (t that product, u the block's sum of the activations) and
 * multiplied by the block's fp16 scale. An MXFP4 code times its power-of-two
 * scale is exact in bf16.
 *
 * x        device [T, H] (dtype as for moe_route)   perm_src device int32 [T*k]
 * work     HOST array of n_work items {expert, slot, row_begin, rows}; items
 *          must not overlap in rows; rows >= 0
 * slot_base device base of the expert blobs; slot_stride bytes between slots
 * wfmt     MOE_W_F32 (x fp32), MOE_W_BF16, MOE_W_INT4 or MOE_W_MXFP4 (x bf16);
 *          the tiled GEMM (MOE_FFN_PREFILL) takes bf16 weights (H % 128,
 *          I % 64 == 0) and MXFP4 weights (H % 256 == 0); AUTO runs the
 *          matrix-vector kernels for the other formats
 * y_perm   device out fp32 [rows_total, H] (only listed rows are written)
 * workspace device scratch, >= moe_ffn_workspace_size(rows_total, H, I, wfmt)
 *          bytes, where rows_total bounds every row index used
 * mode     MOE_FFN_AUTO picks the matrix-vector kernels when every group has
 *          at most 32 rows and the tiled matrix-core GEMM otherwise.
 * Errors: MOE_EINVAL for null pointers, unsupported shapes or formats.
 * ------------------------------------------------------------------------ */
typedef struct { int32_t expert, slot, row_begin, rows; } moe_work_t;

size_t moe_ffn_workspace_size(int rows_total, int H, int I, int wfmt);
int moe_ffn(const void* x, int dtype, const int32_t* perm_src,
            const moe_work_t* work, int n_work,
            const void* slot_base, size_t slot_stride, int wfmt, int H, int I,
            float* y_perm, void* workspace, size_t ws_bytes, int mode, void* stream);

/* moe_ffn_grouped: the same computation for every expert e in 0..E-1 with
 * counts[e] > 0, its group being rows offsets[e] .. offsets[e]+counts[e]-1 of
 * the grouped layout, with the work list read from DEVICE memory (counts and
 * offsets as moe_route writes them) and planned on the GPU, so the call
 * neither waits for the GPU nor copies control data (page "FreeToken-rtx-4090",
 * phase table row "Prefill": a layer's experts are computed as a whole once
 * the layer is resident). Always the tiled matrix-core GEMM.
 *   counts  device int32 [E]; offsets device int32 [E+1] (only [0, E) read)
 *   slot_of device int32 [E]: slot of expert e's blob, or NULL for slot e
 *   n_slots slots at slot_base; rows_max bounds every row (e.g. T*k)
 *   wfmt    MOE_W_BF16 (H and 2I multiples of 256, I of 32) or MOE_W_MXFP4
 *           (H % 256 == 0, I % 128 == 0); x bf16 [T, H]
 *   workspace >= moe_ffn_workspace_size(rows_max, H, I, wfmt) bytes
 * A group whose rows reach past rows_max, or whose slot is outside
 * [0, n_slots), is not computed (its rows of y_perm are left as they were).
 * Errors: MOE_EINVAL for null pointers, unsupported shapes or formats, E
 * outside 1..1024; MOE_EHIP if a launch fails. */
int moe_ffn_grouped(const void* x, int dtype, const int32_t* perm_src, const int32_t* counts,
                    const int32_t* offsets, const int32_t* slot_of, int E, int n_slots, int rows_max,
                    const void* slot_base, size_t slot_stride, int wfmt, int H, int I, float* y_perm,
                    void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Weighted combine. Page "FreeToken-rtx-4090", section "How the MoE Memory
 * Hierarchy Works": a token activates a small subset of a layer's routed
 * experts (six of 256 in the model described); the layer's output for the
 * token is their outputs weighted by the router (the pages do not write the
 * sum; the weights are moe_route's renormalised softmax):
 *   out[t, :] = sum_{j=0..k-1} topk_w[t,j] * y_perm[perm_pos[t,j], :]
 * summed in ascending j in fp32 (no atomics: the result is deterministic).
 * y_perm device fp32 [T*k, H]; perm_pos device int32 [T, k]; topk_w device
 * fp32 [T, k]; out device [T, H] of out_dtype (MOE_DT_F32 or MOE_DT_BF16).
 * ------------------------------------------------------------------------ */
int moe_combine(const float* y_perm, const int32_t* perm_pos, const float* topk_w,
                int T, int k, int H, void* out, int out_dtype, void* stream);

/* ------------------------------------------------------------------------ *
 * Prefill double buffering.
 *
 * Page "FreeToken-rtx-4090", phase table row "Prefill" and the paragraph after
 * it, and page "FreeToken-benchmark", section "How FreeToken Serves Large MoE
 * Models": during prefill the next layer's experts stream over PCIe while the
 * GPU computes the current layer.
 *
 * A pipe owns two device buffers of layer_bytes each (allocated at create)
 * and copies layer l's experts (layer_src[l], layer_bytes bytes, pinned host;
 * the array holds n_layers addresses and is copied at create) into buffer
 * l % 2 on its own copy stream.
 * moe_pipe_begin_layer(l, compute_stream): makes compute_stream wait until
 *   layer l is resident (starting its copy if it was not started), then starts
 *   the copy of layer l+1 into the other buffer once the compute of layer l-1
 *   (recorded by moe_pipe_end_layer) has finished with that buffer.
 *   *buffer receives the device address of layer l's experts.
 * moe_pipe_end_layer(l, compute_stream): records that the compute enqueued so
 *   far for layer l is the last reader of its buffer.
 * moe_pipe_copy_ms: elapsed copy time of layer l (valid after its copy ended).
 * Layers must be visited in order 0, 1, ..., n_layers-1.
 * ------------------------------------------------------------------------ */
typedef struct moe_pipe moe_pipe_t;
moe_pipe_t* moe_pipe_create(const void* const* layer_src, size_t layer_bytes, int n_layers, int* status);
int moe_pipe_destroy(moe_pipe_t* pipe);
int moe_pipe_begin_layer(moe_pipe_t* pipe, int layer, void* compute_stream, void** buffer);
int moe_pipe_end_layer(moe_pipe_t* pipe, int layer, void* compute_stream);
int moe_pipe_copy_ms(moe_pipe_t* pipe, int layer, float* ms);

/* ------------------------------------------------------------------------ *
 * Clock diagnostic of the prefill expert GEMMs.
 *
 * Matrix-core throughput is quoted against the datasheet peak at 2.4 GHz; under
 * sustained matrix-core load the shader clock drops below that (power limit),
 * so a second figure against the peak at the clock the kernels actually ran
 * at needs that clock. moe_clock_record(sums): sums is a device pointer to two
 * uint64 (the caller zeroes them) or NULL (off). While it is set, every block
 * of the prefill expert GEMM launches (moe_ffn in prefill mode, bf16 and
 * MXFP4 weights; not the router) adds the shader-clock cycles and the 100 MHz
 * real-time ticks it spent from its start to the end of its main loop to
 * sums[0] and sums[1] with device atomics, so sums[0] / sums[1] * 0.1 is the
 * time-weighted mean clock in GHz. The setting is process-wide and read when
 * a launch is enqueued: set it while no other thread enqueues prefill work,
 * keep the buffer alive until those launches have finished. Returns MOE_OK.
 * ------------------------------------------------------------------------ */
int moe_clock_record(unsigned long long* sums);

/* ------------------------------------------------------------------------ *
 * Decode layer-step driver.
 *
 * One call runs a whole decode layer-step -- moe_route, the copy of the
 * per-expert counts to the host (the only device-to-host round trip),
 * cache_resolve, cache_fill_async for each wave's misses on the decoder's own
 * fill stream, moe_ffn for each wave, moe_combine -- with the semantics of
 * those calls. Page "FreeToken-rtx-4090", phase table row "Decode" (the
 * shared LRU cache) and component table rows "GPU memory" and "PCIe link".
 *
 * moe_decoder_create: `cache` is used (not owned); blob `key` is at
 *   layer_pool[key / E] + (key % E)*blob_stride (pinned host; the array of the
 *   cache's L layer addresses is copied); slots at slot_base + slot*slot_stride
 *   (device). `buffers` are caller-owned device buffers sized for T_max tokens:
 *   topk_idx int32 [T_max,k], topk_w fp32 [T_max,k], logits fp32 [T_max,E] or
 *   NULL, counts int32 [E], offsets int32 [E+1], perm_src int32 [T_max*k],
 *   perm_pos int32 [T_max,k], y_perm fp32 [T_max*k,H], route_ws of at least
 *   moe_route_workspace_size(T_max,H,E,k) bytes and ffn_ws of at least
 *   moe_ffn_workspace_size(T_max*k,H,I,wfmt) bytes. After a step they hold
 *   that step's routing.
 * moe_decoder_step: x [T,H] (dtype), Wr [H,E], bias [E] or NULL, out [T,H] of
 *   out_dtype; *n_miss (nullable) = fills issued. Blocks the calling thread
 *   until the counts reach the host; the rest is enqueued on `stream`.
 *   On a failed fill the affected keys are invalidated (never half-resident).
 *   The hits' FFN never waits for the misses' copies; each wave's misses'
 *   FFN follows that wave's copies (page "FreeToken-rtx-4090": transfers
 *   overlap computation instead of each expert movement being waited for).
 *   For T <= 16 the decoder keeps a copy of the cache's slot table in device
 *   memory: right after the routing a kernel lists the layer-step's experts
 *   that the copy shows as resident and their FFN is enqueued at once,
 *   before the counts reach the host; the host's resolve then checks that
 *   they are exactly its hits (MOE_EHIP if not) and the copy takes the
 *   step's fills. The copy is uploaded again whole after any change to the
 *   cache made other than through this decoder's resolve (invalidation,
 *   resize); such a change must not happen while a step is being enqueued.
 *   For T > 16 the hits' FFN of each wave is enqueued after the resolve and
 *   before the stream waits for the wave's fills. With bf16 weights, at most
 *   8 experts in the step (min(E, k*T) <= 8) and I a multiple of 512 up to
 *   2048, the resident experts' down projection also writes `out` when no
 *   expert of the step is missing (the combine's sum, in its order), and no
 *   combine is launched; y_perm still receives every row. Otherwise (bf16,
 *   int4 and MXFP4 weights) the resident experts' two projections run as one
 *   launch whose down-projection blocks wait, through flags the decoder
 *   owns, for their expert's gate/up blocks (so one decoder's steps must
 *   stay ordered on one stream).
 *   out_dtype other than MOE_DT_F32 / MOE_DT_BF16 is MOE_EINVAL.
 *   When the cache splits misses (moe_cache_set_split), the misses assigned
 *   to the CPU run with moe_cpu_ffn from the pool on the calling thread while
 *   the GPU works on the others (bf16 activations with bf16, int4 or MXFP4
 *   weights, else MOE_EINVAL); their rows of y_perm are copied in before the
 *   combine.
 * moe_decoder_profile: every > 0 brackets every every-th FFN call of a
 *   layer-step whose experts were all resident (one wave, no fills; the
 *   first such call, then each every-th after it) with HIP events on
 *   `stream`; 0 turns it off;
 *   negative is EINVAL. moe_decoder_ffn_stats returns, over the bracketed
 *   calls since profiling was last set, the summed algorithmic bytes (expert
 *   blobs read + activations read/written), the summed milliseconds and the
 *   number of bracketed calls.
 * moe_decoder_fills: total fills issued by this decoder.
 * moe_decoder_cpu_runs: total misses this decoder ran on the CPU.
 * moe_decoder_resize: moe_cache_resize on the decoder's cache, plus the blob
 *   copies on `stream` (ordered after the decoder's earlier steps on it):
 *   each move, and when slot_base is not NULL (a new caller-owned buffer of at
 *   least S_new * slot_stride bytes) every kept entry into it; the decoder
 *   then uses that buffer (free the old one once the stream has passed the
 *   copies). slot_base NULL keeps the buffer, which must then hold S_new
 *   slots. Errors as moe_cache_resize, EHIP.
 * ------------------------------------------------------------------------ */
typedef struct moe_decoder moe_decoder_t;
typedef struct {
  int32_t* topk_idx;
  float* topk_w;
  float* logits;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_src;
  int32_t* perm_pos;
  float* y_perm;
  void* route_ws;
  size_t route_ws_bytes;
  void* ffn_ws;
  size_t ffn_ws_bytes;
} moe_decoder_buffers_t;

moe_decoder_t* moe_decoder_create(moe_cache_t* cache, int T_max, int H, int I, int E, int k, int dtype, int wfmt,
                                  const void* const* layer_pool, size_t blob_stride, void* slot_base,
                                  size_t slot_stride,
                                  const moe_decoder_buffers_t* buffers, int* status);
int moe_decoder_destroy(moe_decoder_t* decoder);
int moe_decoder_step(moe_decoder_t* decoder, int step, int layer, const void* x, int T, const void* Wr,
                     const float* bias, void* out, int out_dtype, void* stream, int* n_miss);
int moe_decoder_profile(moe_decoder_t* decoder, int every);
int moe_decoder_ffn_stats(moe_decoder_t* decoder, double* bytes, double* ms, int64_t* launches);
int moe_decoder_fills(const moe_decoder_t* decoder, int64_t* fills);
int moe_decoder_cpu_runs(const moe_decoder_t* decoder, int64_t* runs);
int moe_decoder_resize(moe_decoder_t* decoder, int S_new, void* slot_base, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill layer.
 *
 * Page "FreeToken-rtx-4090", phase table row "Prefill" and the paragraph after
 * it: prefill activates a broad part of a layer's experts, and the layer is
 * computed from a buffer holding all of them (a moe_pipe buffer or any
 * resident copy). One call enqueues, on `stream`, moe_route, moe_ffn_grouped
 * with the routing's device counts and offsets (expert e's blob at
 * layer_base + e*blob_stride) and moe_combine into `out` [T, H] (out_dtype);
 * nothing waits for the GPU, copies control data or allocates. `b` holds the
 * caller's device buffers as for moe_decoder_create, sized for T tokens
 * (logits may be NULL); after the call they hold the layer's routing and
 * y_perm. Requirements and errors as moe_route and moe_ffn_grouped (bf16
 * activations; bf16 or MXFP4 experts).
 * ------------------------------------------------------------------------- */
int moe_prefill_layer(const void* x, int dtype, const void* Wr, const float* bias, int T, int H, int E, int k,
                      int I, int wfmt, const void* layer_base, size_t blob_stride, const moe_decoder_buffers_t* b,
                      void* out, int out_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * CPU execution of an expert (page "FreeToken-rtx-4090", component table row
 * "CPU" and section "Adaptive Misses"; page "FreeToken-benchmark", "Adaptive
 * Misses"): a missing expert may run on the host straight from the pinned
 * pool instead of being copied to the GPU.
 *
 * moe_cpu_ffn: y = (silu(x W1) * (x W3)) W2 for `rows` activation rows, on the
 *   host CPU, from the expert's blob (the moe_pack_expert layout) in bf16,
 *   int4 or MXFP4. The 4-bit formats are read as the GPU reads them: int4
 *   codes enter bf16 dot products as 1 + n/16 and each 128-row block's sum
 *   is 16 t - 24 u (u: the activations' sum over the block) times its fp16
 *   scale; MXFP4 codes enter as their E2M1 values and the E8M0 scale
 *   multiplies each 32-row partial sum.
 *   blob: host pointer (e.g. inside a moe_pool_alloc region); x: host bf16
 *   [rows, H] row-major; y: host fp32 [rows, H] row-major, overwritten. The
 *   SwiGLU product is rounded to bf16 before the down projection, as on the
 *   GPU. threads: participating threads (<= 0: all, see moe_cpu_threads);
 *   the library keeps one process-wide pool of worker threads, and calls from
 *   several host threads at once are serialised by the caller. Synchronous.
 *   Errors: EINVAL for null pointers, negative rows, fp32 weights, or H, I
 *   not multiples of 32 (bf16) or 128 (int4, MXFP4). Needs a CPU with
 *   AVX-512 BF16.
 * moe_cpu_threads: the number of threads moe_cpu_ffn can use (workers + the
 *   calling thread).
 * ------------------------------------------------------------------------- */
int moe_cpu_ffn(const void* blob, int wfmt, int H, int I, const void* x, int rows, float* y, int threads);
int moe_cpu_threads(void);

/* ---------------------------------------------------------------------------
 * Device-controlled decode layer-step and graph capture.
 *
 * Page "FreeToken-benchmark", section "Graph Compatibility": routing-dependent
 * decisions are kept in device-resident control data so that the decode step
 * can run as captured, replayable GPU work. Here every decision of the step
 * (which experts, hit or miss, which slot, which victim) is made by kernels
 * from tables in GPU memory; the host only enqueues.
 *
 * moe_device_decoder_create: an L-layer cache of S slots with the policy of
 *   cache_resolve (hits ascending, then misses ascending; lowest free slot,
 *   else least recently used), its state held in GPU memory (allocated and
 *   owned by the decoder; the cache starts empty). Every miss is filled (there
 *   is no CPU execution on this path). Requires S >= min(E, k*T_max), so that
 *   a layer-step's experts always fit the cache at once (one wave), and
 *   E <= 1024. layer_pool: the L per-layer base addresses of moe_pool_alloc
 *   memory (host; layers may share a base), read over the host link by the
 *   FFN (fp32 experts: by the fill kernel). slot_base/slot_stride, buffers
 *   and the other arguments as for moe_decoder_create (the decoder never
 *   frees them). trace_capacity: number of trace records kept in GPU memory
 *   (0: none).
 *   Errors: EINVAL (null, bad sizes, pool address not from moe_pool_alloc),
 *   ECAPACITY (S too small), ENOMEM (device memory), EHIP.
 * moe_device_decoder_step: enqueues one layer-step on `stream`: routing (as
 *   moe_route), the resolve (one workgroup updates the tables and writes the
 *   work list, hits first, and the number of hits to GPU memory; for T <= 16
 *   it runs at the end of the routing launch's last kernel, else as a kernel
 *   of its own),
 *   the decode expert FFN over the device work list (fixed grid for
 *   min(E, k*T) items; surplus blocks exit) and the combine into `out` (for
 *   bf16 weights with min(E, k*T) <= 8 and I a multiple of 512 up to 2048,
 *   formed by the down projection itself, with no combine launch). For
 *   bf16, int4 and MXFP4 experts the FFN reads each hit from its slot and
 *   each miss from the pool over the host link, writing the miss's blob
 *   through into its slot as it goes (the fill; both projections run as one
 *   launch, numbered by the resolve's call counter, unless the down
 *   projection forms `out`);
 *   for fp32 experts a fill
 *   kernel first copies the misses' blobs into their slots (returning at once
 *   when there are none) and the FFN then reads every item from its slot.
 *   It neither waits for the GPU nor allocates, so the same call can be
 *   captured with moe_graph_begin/moe_graph_end and replayed: a replay reads
 *   whatever x, Wr and bias hold at that time. Launch shapes depend only on
 *   T, so a graph is tied to the T (and layer and buffers) it was captured
 *   with. Steps on one decoder must run in stream order (one stream, or
 *   explicit ordering). Errors: EINVAL (null, T or layer out of range), EHIP.
 * moe_device_decoder_stats: total hits, misses (= fills) and resolve calls.
 * moe_device_decoder_trace: copies up to max_records trace records (the
 *   first trace_capacity accesses since the last clear, access order) and
 *   sets *n_records to the number of accesses traced since then (may exceed
 *   the capacity). Records are as moe_trace_t with step = the sequence number
 *   of the resolve call that made them (0, 1, ... from creation) and wave 0.
 * moe_device_decoder_resize: the resize of moe_cache_resize (same kept
 *   entries, slots and moves) on the device tables: waits for `stream` (the
 *   safe point), plans on the host, copies the blobs as moe_decoder_resize
 *   does, rewrites the tables (reallocated when S changes), and waits again.
 *   S_new must stay >= min(E, k*T_max). Graphs captured before a resize read
 *   the old tables and buffer: capture again. Errors: ECAPACITY, EHIP, ENOMEM.
 * moe_device_decoder_clear_trace, moe_device_decoder_slot_of: as for the host
 *   cache. stats, trace and slot_of read GPU memory with blocking copies: call
 *   them once the stream's steps have completed.
 *
 * moe_graph_begin(stream): starts capturing `stream` (a created stream, not
 *   the default one; thread-local capture mode). moe_graph_end(stream): ends
 *   the capture and instantiates it. moe_graph_launch: replays the graph on a
 *   stream. moe_graph_destroy frees it. Errors: EINVAL, EHIP (for example a
 *   call that is not allowed during capture).
 * ------------------------------------------------------------------------- */
typedef struct moe_device_decoder moe_device_decoder_t;
typedef struct moe_graph moe_graph_t;

moe_device_decoder_t* moe_device_decoder_create(int L, int E, int S, int T_max, int H, int I, int k, int dtype,
                                                int wfmt, const void* const* layer_pool, size_t blob_stride,
                                                void* slot_base, size_t slot_stride,
                                                const moe_decoder_buffers_t* buffers, int64_t trace_capacity,
                                                int* status);
int moe_device_decoder_destroy(moe_device_decoder_t* decoder);
int moe_device_decoder_step(moe_device_decoder_t* decoder, int layer, const void* x, int T, const void* Wr,
                            const float* bias, void* out, int out_dtype, void* stream);
int moe_device_decoder_stats(const moe_device_decoder_t* decoder, int64_t* hits, int64_t* misses,
                             int64_t* resolves);
int moe_device_decoder_trace(const moe_device_decoder_t* decoder, moe_trace_t* out, int64_t max_records,
                             int64_t* n_records);
int moe_device_decoder_clear_trace(moe_device_decoder_t* decoder);
int moe_device_decoder_slot_of(const moe_device_decoder_t* decoder, int key, int* slot);
int moe_device_decoder_resize(moe_device_decoder_t* decoder, int S_new, void* slot_base, void* stream);

int moe_graph_begin(void* stream);
moe_graph_t* moe_graph_end(void* stream, int* status);
int moe_graph_launch(moe_graph_t* graph, void* stream);
int moe_graph_destroy(moe_graph_t* graph);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
