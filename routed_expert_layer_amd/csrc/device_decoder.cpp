// Device-controlled decode layer-step: routing, cache resolve, fills, expert
// FFN and combine enqueued on one stream with every routing-dependent choice
// made by kernels from device-resident tables, so the step never waits for
// the host and can be captured into a HIP graph and replayed (page
// "FreeToken-benchmark", section "Graph Compatibility"). The cache policy is
// the shared LRU of the host path (page "FreeToken-rtx-4090", section "How the
// MoE Memory Hierarchy Works"); misses are always filled (the CPU share of
// "Adaptive Misses" needs the host and stays on the host-driven path).
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "../../include/moe.h"
#include "lru_policy.hpp"
#include "moe_kernels.hpp"

extern "C" size_t moe_route_workspace_size(int T, int H, int E, int k);

namespace {
template <typename... A>
int dd_fail(int code, const char* fmt, A... a) {
  return moe::set_error(code, fmt, a...);
}
}  // namespace

struct moe_device_decoder {
  int L, E, S, Tmax, H, I, k, dtype, wfmt;
  std::vector<const char*> pool;  // device-visible address of each layer's pool
  size_t blob_stride, blob_bytes;
  char* slot_base;
  size_t slot_stride;
  moe_decoder_buffers_t b;
  void* mem = nullptr;  // one device allocation holding the control data
  moe::DevCache c{};
  int max_items;
  uint64_t* ffn_flags = nullptr;  // hand-off flags of the one-launch FFN (zeroed at creation)
};

namespace {
// Offsets of the control data in its allocation (256-byte aligned pieces).
struct CtlLayout {
  size_t slot_of, slot_key, stamp, ctl, work, miss, n, trace, total;
};
CtlLayout ctl_layout(size_t n_keys, int S, int max_items, int64_t trace_cap) {
  CtlLayout o{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = moe::align_up(off + bytes, 256);
    return at;
  };
  o.slot_of = take(n_keys * 4);
  o.slot_key = take((size_t)S * 4);
  o.stamp = take((size_t)S * 8);
  o.ctl = take(8 * 8);
  o.work = take((size_t)max_items * 16);
  o.miss = take((size_t)max_items * 16);
  o.n = take(3 * 4);
  o.trace = take((size_t)trace_cap * 7 * 4);
  o.total = off;
  return o;
}
void point_into(moe::DevCache& c, char* m, const CtlLayout& o, int S, int64_t trace_cap) {
  c.slot_of = reinterpret_cast<int32_t*>(m + o.slot_of);
  c.slot_key = reinterpret_cast<int32_t*>(m + o.slot_key);
  c.stamp = reinterpret_cast<uint64_t*>(m + o.stamp);
  c.ctl = reinterpret_cast<uint64_t*>(m + o.ctl);
  c.S = S;
  c.work = reinterpret_cast<int4*>(m + o.work);
  c.miss = reinterpret_cast<int4*>(m + o.miss);
  c.n = reinterpret_cast<int32_t*>(m + o.n);
  c.trace = reinterpret_cast<int32_t*>(m + o.trace);
  c.trace_cap = trace_cap;
}
}  // namespace

struct moe_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" {

static void dd_release(moe_device_decoder_t* d) {
  if (d->mem) (void)hipFree(d->mem);
  if (d->ffn_flags) (void)hipFree(d->ffn_flags);
  delete d;
}

moe_device_decoder_t* moe_device_decoder_create(int L, int E, int S, int T_max, int H, int I, int k, int dtype,
                                                int wfmt, const void* const* layer_pool, size_t blob_stride,
                                                void* slot_base, size_t slot_stride,
                                                const moe_decoder_buffers_t* buffers, int64_t trace_capacity,
                                                int* status) {
  auto bad = [&](int code, const char* msg) -> moe_device_decoder_t* {
    if (status) *status = dd_fail(code, "moe_device_decoder_create: %s", msg);
    return nullptr;
  };
  if (!layer_pool || !slot_base || !buffers) return bad(MOE_EINVAL, "null argument");
  if (L < 1 || E < 1 || E > 1024 || (long long)L * E > (1ll << 30) || T_max < 1 || H < 1 || I < 1 || k < 1 ||
      k > 16 || k > E || H % 8 != 0 || trace_capacity < 0)
    return bad(MOE_EINVAL, "bad sizes");
  if (S < 1) return bad(MOE_ECAPACITY, "the cache needs at least one slot");
  const int max_items = E < k * T_max ? E : k * T_max;
  if (S < max_items)
    return bad(MOE_ECAPACITY, "S must be at least min(E, k*T_max): a layer-step's experts must fit the cache at once");
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return bad(MOE_EINVAL, "bad activation dtype");
  if ((wfmt == MOE_W_F32) != (dtype == MOE_DT_F32)) return bad(MOE_EINVAL, "activation dtype does not match weights");
  const size_t blob = moe_expert_bytes(wfmt, H, I);
  if (blob == 0) return bad(MOE_EINVAL, "unsupported weight format or shape");
  if (blob % 16 != 0) return bad(MOE_EINVAL, "expert blob size not a multiple of 16 bytes");
  if (blob_stride < blob || slot_stride < blob) return bad(MOE_EINVAL, "stride smaller than an expert blob");
  const moe_decoder_buffers_t& b = *buffers;
  if (!b.topk_idx || !b.topk_w || !b.counts || !b.offsets || !b.perm_src || !b.perm_pos || !b.y_perm ||
      !b.route_ws || !b.ffn_ws)
    return bad(MOE_EINVAL, "null device buffer");
  if (b.route_ws_bytes < moe_route_workspace_size(T_max, H, E, k)) return bad(MOE_EINVAL, "route workspace too small");
  if (b.ffn_ws_bytes < moe_ffn_workspace_size(T_max * k, H, I, wfmt)) return bad(MOE_EINVAL, "FFN workspace too small");
  moe_device_decoder_t* d = new (std::nothrow) moe_device_decoder();
  if (!d) return bad(MOE_ENOMEM, "out of host memory");
  d->L = L; d->E = E; d->S = S; d->Tmax = T_max; d->H = H; d->I = I; d->k = k; d->dtype = dtype; d->wfmt = wfmt;
  d->blob_stride = blob_stride; d->blob_bytes = blob;
  d->slot_base = static_cast<char*>(slot_base);
  d->slot_stride = slot_stride;
  d->b = b;
  d->max_items = max_items;
  for (int l = 0; l < L; ++l) {
    void* dp = nullptr;
    if (!layer_pool[l] || hipHostGetDevicePointer(&dp, const_cast<void*>(layer_pool[l]), 0) != hipSuccess || !dp) {
      dd_release(d);
      return bad(MOE_EINVAL, "a layer pool address is not pinned host memory from moe_pool_alloc");
    }
    d->pool.push_back(static_cast<const char*>(dp));
  }
  // control data, 256-byte aligned pieces of one allocation
  const CtlLayout o = ctl_layout((size_t)L * E, S, max_items, trace_capacity);
  hipError_t e = hipMalloc(&d->mem, o.total);
  if (e != hipSuccess) {
    d->mem = nullptr;
    dd_release(d);
    if (status) *status = dd_fail(MOE_ENOMEM, "moe_device_decoder_create: %s", hipGetErrorString(e));
    return nullptr;
  }
  point_into(d->c, static_cast<char*>(d->mem), o, S, trace_capacity);
  char* m = static_cast<char*>(d->mem);
  // empty cache: every key unmapped (-1 bytes), every slot free, clocks zero
  e = hipMemset(m + o.slot_of, 0xFF, o.stamp - o.slot_of);
  if (e == hipSuccess) e = hipMemset(m + o.stamp, 0, o.trace - o.stamp);
  if (e == hipSuccess && moe::ffn_fused_ok(wfmt, H, I)) {
    const size_t fb = sizeof(uint64_t) * moe::ffn_fused_flags(max_items, I);
    e = hipMalloc(reinterpret_cast<void**>(&d->ffn_flags), fb);
    if (e == hipSuccess) e = hipMemset(d->ffn_flags, 0, fb);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    dd_release(d);
    if (status) *status = dd_fail(MOE_EHIP, "moe_device_decoder_create: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (status) *status = MOE_OK;
  return d;
}

int moe_device_decoder_destroy(moe_device_decoder_t* d) {
  if (!d) return MOE_OK;
  (void)hipDeviceSynchronize();
  dd_release(d);
  return MOE_OK;
}

int moe_device_decoder_step(moe_device_decoder_t* d, int layer, const void* x, int T, const void* Wr,
                            const float* bias, void* out, int out_dtype, void* stream) {
  if (!d || !x || !Wr || !out) return dd_fail(MOE_EINVAL, "moe_device_decoder_step: null argument");
  if (T < 1 || T > d->Tmax) return dd_fail(MOE_EINVAL, "moe_device_decoder_step: T=%d outside [1, %d]", T, d->Tmax);
  if (layer < 0 || layer >= d->L) return dd_fail(MOE_EINVAL, "moe_device_decoder_step: layer %d out of range", layer);
  if (out_dtype != MOE_DT_F32 && out_dtype != MOE_DT_BF16)
    return dd_fail(MOE_EINVAL, "moe_device_decoder_step: bad output dtype");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const moe_decoder_buffers_t& b = d->b;
  const int items = d->E < d->k * T ? d->E : d->k * T;
  char* ws = static_cast<char*>(b.ffn_ws);
  void* hbuf = ws;
  // decode-size batches: the routing launch's last kernel also runs the resolve (one launch fewer)
  const bool fused_resolve = moe::route_small_path(T, d->E);
  // bf16 steps of few experts: the down projection forms `out` itself (no combine launch)
  const bool fused_combine = moe::ffn_combine_ok(d->wfmt, d->H, d->I, items, T, d->k);
  const moe::DevStep dstep{d->c, layer};
  hipError_t e = moe::launch_route(x, d->dtype == MOE_DT_BF16, Wr, bias, T, d->H, d->E, d->k, b.topk_idx, b.topk_w,
                                   b.logits, b.counts, b.offsets, b.perm_src, b.perm_pos, b.route_ws, s, nullptr, 0,
                                   nullptr, fused_resolve ? &dstep : nullptr);
  if (e == hipSuccess && !fused_resolve) e = moe::launch_dev_resolve(b.counts, b.offsets, d->E, layer, d->c, s);
  if (d->wfmt == MOE_W_F32) {
    // fp32 experts: the misses are copied first, then every item runs from its slot
    if (e == hipSuccess)
      e = moe::launch_dev_fill(d->c, d->pool[layer], d->blob_stride, d->blob_bytes, d->slot_base, d->slot_stride, s);
    if (e == hipSuccess)
      e = moe::launch_ffn_decode_dev(d->wfmt, x, b.perm_src, d->c.n, d->c.work, items, T, d->slot_base,
                                     d->slot_stride, d->H, d->I, hbuf, b.y_perm, s);
  } else if (e == hipSuccess && fused_combine) {
    // the same pass, with the down projection also forming `out` (every expert of the step is in the list)
    e = moe::launch_ffn_decode_combine(x, b.perm_src, d->c.n, d->c.work, items, T, d->slot_base, d->slot_stride, d->H,
                                       d->I, hbuf, b.y_perm, d->c.n, b.perm_pos, b.topk_w, d->k, out,
                                       out_dtype == MOE_DT_BF16, s, d->c.n + 2, d->pool[layer], d->blob_stride);
  } else if (e == hipSuccess && d->ffn_flags != nullptr) {
    // the same pass with both projections in one launch; the resolve's call counter numbers the calls
    e = moe::launch_ffn_decode_fused(d->wfmt, x, b.perm_src, d->c.n, d->c.work, items, d->slot_base, d->slot_stride,
                                     d->H, d->I, hbuf, b.y_perm, d->ffn_flags, 0, s, d->c.ctl + 3, d->c.n + 2,
                                     d->pool[layer], d->blob_stride);
  } else if (e == hipSuccess) {
    // one pass: the hits run from their slots while the misses stream from the pool over the host link and
    // are written through into their slots
    e = moe::launch_ffn_decode_dev(d->wfmt, x, b.perm_src, d->c.n, d->c.work, items, T, d->slot_base, d->slot_stride,
                                   d->H, d->I, hbuf, b.y_perm, s, d->c.n + 2, d->pool[layer], d->blob_stride);
  }
  if (e == hipSuccess && !fused_combine)
    e = moe::launch_combine(b.y_perm, b.perm_pos, b.topk_w, T, d->k, d->H, out, out_dtype == MOE_DT_BF16, s);
  if (e != hipSuccess) return dd_fail(MOE_EHIP, "moe_device_decoder_step: %s", hipGetErrorString(e));
  return MOE_OK;
}

int moe_device_decoder_resize(moe_device_decoder_t* d, int S_new, void* slot_base, void* stream) {
  if (!d) return dd_fail(MOE_EINVAL, "moe_device_decoder_resize: null decoder");
  if (S_new < d->max_items)
    return dd_fail(MOE_ECAPACITY, "moe_device_decoder_resize: S must stay at least min(E, k*T_max) = %d",
                   d->max_items);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // safe point: every step enqueued so far has finished
  hipError_t e = hipStreamSynchronize(s);
  const int S_old = d->S;
  const size_t n_keys = (size_t)d->L * d->E;
  std::vector<int32_t> slot_key(S_old);
  std::vector<uint64_t> stamp(S_old);
  if (e == hipSuccess) e = hipMemcpy(slot_key.data(), d->c.slot_key, (size_t)S_old * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(stamp.data(), d->c.stamp, (size_t)S_old * 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return dd_fail(MOE_EHIP, "moe_device_decoder_resize: %s", hipGetErrorString(e));
  std::vector<int32_t> new_key, origin, evicted;
  std::vector<moe::Move> moves;
  moe::plan_resize(slot_key, stamp, S_new, new_key, origin, moves, evicted);
  std::vector<uint64_t> new_stamp(S_new, 0);
  std::vector<int32_t> slot_of(n_keys, -1);
  for (int sl = 0; sl < S_new; ++sl)
    if (origin[sl] >= 0) {
      new_stamp[sl] = stamp[origin[sl]];
      slot_of[new_key[sl]] = sl;
    }
  // the blobs: moved entries, and every kept entry when the buffer changes
  char* old_base = d->slot_base;
  char* new_base = slot_base ? static_cast<char*>(slot_base) : old_base;
  for (int sl = 0; sl < S_new && e == hipSuccess; ++sl)
    if (origin[sl] >= 0 && (origin[sl] != sl || new_base != old_base))
      e = hipMemcpyAsync(new_base + (size_t)sl * d->slot_stride, old_base + (size_t)origin[sl] * d->slot_stride,
                         d->blob_bytes, hipMemcpyDeviceToDevice, s);
  // the tables, in a new allocation when the slot count changes
  void* mem = d->mem;
  const CtlLayout o_old = ctl_layout(n_keys, S_old, d->max_items, d->c.trace_cap);
  const CtlLayout o_new = ctl_layout(n_keys, S_new, d->max_items, d->c.trace_cap);
  if (e == hipSuccess && S_new != S_old) {
    e = hipMalloc(&mem, o_new.total);
    if (e != hipSuccess) return dd_fail(MOE_ENOMEM, "moe_device_decoder_resize: %s", hipGetErrorString(e));
    // counters, work lists and trace keep their contents
    e = hipMemcpyAsync(static_cast<char*>(mem) + o_new.ctl, static_cast<char*>(d->mem) + o_old.ctl,
                       o_old.total - o_old.ctl, hipMemcpyDeviceToDevice, s);
  }
  char* m = static_cast<char*>(mem);
  if (e == hipSuccess) e = hipMemcpyAsync(m + o_new.slot_of, slot_of.data(), n_keys * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m + o_new.slot_key, new_key.data(), (size_t)S_new * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m + o_new.stamp, new_stamp.data(), (size_t)S_new * 8, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // host vectors are read by the copies
  if (e != hipSuccess) {
    if (mem != d->mem) (void)hipFree(mem);
    return dd_fail(MOE_EHIP, "moe_device_decoder_resize: %s", hipGetErrorString(e));
  }
  if (mem != d->mem) {
    (void)hipFree(d->mem);
    d->mem = mem;
  }
  point_into(d->c, m, o_new, S_new, d->c.trace_cap);
  d->S = S_new;
  d->slot_base = new_base;
  return MOE_OK;
}

int moe_device_decoder_stats(const moe_device_decoder_t* d, int64_t* hits, int64_t* misses, int64_t* resolves) {
  if (!d || !hits || !misses || !resolves) return dd_fail(MOE_EINVAL, "moe_device_decoder_stats: null argument");
  uint64_t ctl[5];
  hipError_t e = hipMemcpy(ctl, d->c.ctl, sizeof ctl, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return dd_fail(MOE_EHIP, "moe_device_decoder_stats: %s", hipGetErrorString(e));
  *hits = (int64_t)ctl[1];
  *misses = (int64_t)ctl[2];
  *resolves = (int64_t)ctl[3];
  return MOE_OK;
}

int moe_device_decoder_trace(const moe_device_decoder_t* d, moe_trace_t* out, int64_t max_records,
                             int64_t* n_records) {
  if (!d || !n_records || max_records < 0 || (max_records > 0 && !out))
    return dd_fail(MOE_EINVAL, "moe_device_decoder_trace: null argument");
  uint64_t n = 0;
  hipError_t e = hipMemcpy(&n, d->c.ctl + 4, sizeof n, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return dd_fail(MOE_EHIP, "moe_device_decoder_trace: %s", hipGetErrorString(e));
  *n_records = (int64_t)n;
  int64_t m = (int64_t)n < d->c.trace_cap ? (int64_t)n : d->c.trace_cap;
  if (m > max_records) m = max_records;
  if (m > 0) {
    e = hipMemcpy(out, d->c.trace, (size_t)m * sizeof(moe_trace_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return dd_fail(MOE_EHIP, "moe_device_decoder_trace: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

int moe_device_decoder_clear_trace(moe_device_decoder_t* d) {
  if (!d) return dd_fail(MOE_EINVAL, "moe_device_decoder_clear_trace: null decoder");
  const uint64_t zero = 0;
  hipError_t e = hipMemcpy(d->c.ctl + 4, &zero, sizeof zero, hipMemcpyHostToDevice);
  return e == hipSuccess ? MOE_OK : dd_fail(MOE_EHIP, "moe_device_decoder_clear_trace: %s", hipGetErrorString(e));
}

int moe_device_decoder_slot_of(const moe_device_decoder_t* d, int key, int* slot) {
  if (!d || !slot || key < 0 || (long long)key >= (long long)d->L * d->E)
    return dd_fail(MOE_EINVAL, "moe_device_decoder_slot_of: bad argument");
  hipError_t e = hipMemcpy(slot, d->c.slot_of + key, sizeof(int32_t), hipMemcpyDeviceToHost);
  return e == hipSuccess ? MOE_OK : dd_fail(MOE_EHIP, "moe_device_decoder_slot_of: %s", hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Stream capture into a HIP graph
// ---------------------------------------------------------------------------
int moe_graph_begin(void* stream) {
  if (!stream) return dd_fail(MOE_EINVAL, "moe_graph_begin: capture needs a created stream, not the default one");
  hipError_t e = hipStreamBeginCapture(reinterpret_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal);
  return e == hipSuccess ? MOE_OK : dd_fail(MOE_EHIP, "moe_graph_begin: %s", hipGetErrorString(e));
}

moe_graph_t* moe_graph_end(void* stream, int* status) {
  auto bad = [&](int code, const char* what, hipError_t e) -> moe_graph_t* {
    if (status) *status = dd_fail(code, "moe_graph_end: %s: %s", what, hipGetErrorString(e));
    return nullptr;
  };
  if (!stream) {
    if (status) *status = dd_fail(MOE_EINVAL, "moe_graph_end: null stream");
    return nullptr;
  }
  moe_graph_t* g = new (std::nothrow) moe_graph();
  if (!g) return bad(MOE_ENOMEM, "allocation", hipSuccess);
  hipError_t e = hipStreamEndCapture(reinterpret_cast<hipStream_t>(stream), &g->graph);
  if (e != hipSuccess || !g->graph) {
    delete g;
    return bad(MOE_EHIP, "end of capture", e);
  }
  e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g->graph);
    delete g;
    return bad(MOE_EHIP, "instantiate", e);
  }
  if (status) *status = MOE_OK;
  return g;
}

int moe_graph_launch(moe_graph_t* g, void* stream) {
  if (!g) return dd_fail(MOE_EINVAL, "moe_graph_launch: null graph");
  hipError_t e = hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : dd_fail(MOE_EHIP, "moe_graph_launch: %s", hipGetErrorString(e));
}

int moe_graph_destroy(moe_graph_t* g) {
  if (!g) return MOE_OK;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
  return MOE_OK;
}

}  // extern "C"
