// C ABI of the routed expert layer (declared in include/moe.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "lru_policy.hpp"
#include "moe_kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

int moe::set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

struct moe_cache {
  int L, E, S;
  moe::SharedLru lru;
  std::vector<moe_trace_t> trace;
  hipEvent_t ev_war = nullptr, ev_done = nullptr;
  // MOE_DEBUG_POISON_FILLS=1 at creation: every fill first sets its slot's
  // bytes to 0xFF (NaN in bf16, fp32 and the fp16 / E8M0 scales), so a read
  // that is not ordered after the fill shows up as non-finite output.
  bool poison = false;
  moe_cache(int L_, int E_, int S_) : L(L_), E(E_), S(S_), lru(L_ * E_, S_) {
    const char* v = std::getenv("MOE_DEBUG_POISON_FILLS");
    poison = v && v[0] == '1';
  }
};

struct moe_pipe {
  std::vector<const char*> src;
  size_t bytes;
  int L;
  void* buf[2] = {nullptr, nullptr};
  hipStream_t copy = nullptr;
  std::vector<hipEvent_t> copied, started, done;
  int next_copy = 0;   // next layer whose copy has not been enqueued
  int next_begin = 0;  // next layer expected by begin_layer
  int next_end = 0;    // next layer expected by end_layer
};

// Internal accessors for the decode driver (C++ linkage).
int moe_cache_layers(const moe_cache_t* c, int* n_layers) {
  if (!c || !n_layers) return MOE_EINVAL;
  *n_layers = c->L;
  return MOE_OK;
}
int moe_cache_experts(const moe_cache_t* c) { return c ? c->E : -1; }
bool moe_cache_splits(const moe_cache_t* c) { return c && c->lru.splits(); }
uint64_t moe_cache_edits(const moe_cache_t* c) { return c ? c->lru.edits() : 0; }

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_abi_version(void) { return 1; }

// ---------------------------------------------------------------------------
// Routing
// ---------------------------------------------------------------------------
size_t moe_route_workspace_size(int T, int H, int E, int k) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0) return 0;
  return moe::route_workspace_bytes(T, H, E, k);
}

int moe_route(const void* x, int dtype, const void* Wr, const float* bias, int T, int H, int E, int k,
              int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm_src,
              int32_t* perm_pos, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || E > 1024 || k < 1 || k > 16 || k > E || (H % 8) != 0)
    return fail(MOE_EINVAL, "moe_route: unsupported sizes T=%d H=%d E=%d k=%d", T, H, E, k);
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "moe_route: bad dtype %d", dtype);
  if (!counts || !offsets || !workspace || (T > 0 && (!x || !Wr || !topk_idx || !topk_w || !perm_src || !perm_pos)))
    return fail(MOE_EINVAL, "moe_route: null pointer argument");
  if (ws_bytes < moe::route_workspace_bytes(T, H, E, k))
    return fail(MOE_EINVAL, "moe_route: workspace too small (%zu < %zu)", ws_bytes,
                moe::route_workspace_bytes(T, H, E, k));
  hipError_t e = moe::launch_route(x, dtype == MOE_DT_BF16, Wr, bias, T, H, E, k, topk_idx, topk_w, logits, counts,
                                   offsets, perm_src, perm_pos, workspace, as_stream(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route launch");
}

// ---------------------------------------------------------------------------
// Blobs and pool
// ---------------------------------------------------------------------------
static bool shape_ok(int wfmt, int H, int I) {
  if (H <= 0 || I <= 0) return false;
  if (wfmt == MOE_W_F32) return true;
  if (wfmt == MOE_W_BF16) return H % 32 == 0 && I % 32 == 0;
  if (wfmt == MOE_W_INT4 || wfmt == MOE_W_MXFP4) return H % 128 == 0 && I % 128 == 0;
  return false;
}

size_t moe_expert_bytes(int wfmt, int H, int I) {
  if (!shape_ok(wfmt, H, I)) return 0;
  return moe::blob_layout(wfmt, H, I).bytes;
}

int moe_pack_expert(int wfmt, int H, int I, const void* W1, const void* W3, const void* W2, const void* s1,
                    const void* s3, const void* s2, void* blob, void* stream) {
  if (!shape_ok(wfmt, H, I)) return fail(MOE_EINVAL, "moe_pack_expert: unsupported format/shape %d %dx%d", wfmt, H, I);
  if (!W1 || !W3 || !W2 || !blob) return fail(MOE_EINVAL, "moe_pack_expert: null pointer argument");
  if ((wfmt == MOE_W_INT4 || wfmt == MOE_W_MXFP4) && (!s1 || !s3 || !s2))
    return fail(MOE_EINVAL, "moe_pack_expert: int4 and MXFP4 need scales");
  hipError_t e = moe::launch_pack(wfmt, H, I, W1, W3, W2, s1, s3, s2, blob, as_stream(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pack_expert");
}

void* moe_pool_alloc(size_t bytes, int* status) {
  void* p = nullptr;
  if (bytes == 0) {
    if (status) *status = fail(MOE_EINVAL, "moe_pool_alloc: zero bytes");
    return nullptr;
  }
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
  if (e != hipSuccess || !p) {
    if (status) *status = fail(MOE_ENOMEM, "moe_pool_alloc(%zu): %s", bytes, hipGetErrorString(e));
    return nullptr;
  }
  moe::cpu_touch_pages(p, bytes);  // CPU execution from the pool pays no first-touch cost later
  if (status) *status = MOE_OK;
  return p;
}

int moe_pool_free(void* pool) {
  if (!pool) return MOE_OK;
  hipError_t e = hipHostFree(pool);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pool_free");
}

// ---------------------------------------------------------------------------
// Cache policy
// ---------------------------------------------------------------------------
moe_cache_t* moe_cache_create(int L, int E, int S, int* status) {
  if (L <= 0 || E <= 0 || (long long)L * E > (1ll << 30)) {
    if (status) *status = fail(MOE_EINVAL, "moe_cache_create: bad L=%d E=%d", L, E);
    return nullptr;
  }
  if (S <= 0) {
    if (status) *status = fail(MOE_ECAPACITY, "moe_cache_create: cache needs at least one slot (S=%d)", S);
    return nullptr;
  }
  moe_cache_t* c = new (std::nothrow) moe_cache(L, E, S);
  if (!c) {
    if (status) *status = fail(MOE_ENOMEM, "moe_cache_create: out of host memory");
    return nullptr;
  }
  if (status) *status = MOE_OK;
  return c;
}

int moe_cache_destroy(moe_cache_t* c) {
  if (!c) return MOE_OK;
  if (c->ev_war) (void)hipEventDestroy(c->ev_war);
  if (c->ev_done) (void)hipEventDestroy(c->ev_done);
  delete c;
  return MOE_OK;
}

int cache_resolve(moe_cache_t* c, int step, int layer, const int32_t* experts, int n, int32_t* work_e,
                  int32_t* work_slot, int32_t* work_wave, moe_miss_t* misses, int* n_miss, int* n_waves) {
  if (!c || n < 0 || (n > 0 && (!experts || !work_e || !work_slot || !work_wave || !misses)) || !n_miss || !n_waves)
    return fail(MOE_EINVAL, "cache_resolve: null pointer or negative count");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "cache_resolve: layer %d out of range [0,%d)", layer, c->L);
  std::vector<int32_t> keys(n);
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= c->E)
      return fail(MOE_EINVAL, "cache_resolve: expert %d out of range [0,%d)", experts[i], c->E);
    if (i > 0 && experts[i] <= experts[i - 1])
      return fail(MOE_EINVAL, "cache_resolve: experts must be ascending and unique");
    keys[i] = layer * c->E + experts[i];
  }
  std::vector<moe::Access> acc;
  acc.reserve(n);
  c->lru.resolve(keys.data(), n, acc);
  int nm = 0, nw = 0;
  for (int i = 0; i < n; ++i) {
    const moe::Access& a = acc[i];
    work_e[i] = a.key - layer * c->E;
    work_slot[i] = a.slot;  // -1: run on the CPU
    work_wave[i] = a.wave;
    nw = std::max(nw, a.wave + 1);
    if (!a.hit && a.slot >= 0) misses[nm++] = moe_miss_t{a.key, a.slot, a.victim, a.wave};
    c->trace.push_back(moe_trace_t{step, layer, a.key, a.hit, a.slot, a.victim, a.wave});
  }
  *n_miss = nm;
  *n_waves = nw;
  return MOE_OK;
}

int moe_cache_set_split(moe_cache_t* c, int rate_gpu, int rate_cpu) {
  if (!c || rate_gpu < 0 || rate_cpu < 0 || rate_gpu + rate_cpu <= 0)
    return fail(MOE_EINVAL, "moe_cache_set_split: rates must be >= 0 with a positive sum");
  c->lru.set_split(rate_gpu, rate_cpu);
  return MOE_OK;
}

int moe_cache_trace(const moe_cache_t* c, moe_trace_t* out, int64_t max_records, int64_t* n_records) {
  if (!c || !n_records || (max_records > 0 && !out)) return fail(MOE_EINVAL, "moe_cache_trace: null pointer");
  const int64_t n = (int64_t)c->trace.size();
  *n_records = n;
  const int64_t m = std::min<int64_t>(n, std::max<int64_t>(max_records, 0));
  if (m > 0) std::memcpy(out, c->trace.data(), (size_t)m * sizeof(moe_trace_t));
  return MOE_OK;
}

int moe_cache_clear_trace(moe_cache_t* c) {
  if (!c) return fail(MOE_EINVAL, "moe_cache_clear_trace: null cache");
  c->trace.clear();
  return MOE_OK;
}

int moe_cache_invalidate(moe_cache_t* c, int key) {
  if (!c || key < 0 || key >= c->L * c->E) return fail(MOE_EINVAL, "moe_cache_invalidate: bad key %d", key);
  if (!c->lru.invalidate(key)) return fail(MOE_EINVAL, "moe_cache_invalidate: key %d not resident", key);
  return MOE_OK;
}

int moe_cache_slot_of(const moe_cache_t* c, int key, int* slot) {
  if (!c || !slot || key < 0 || key >= c->L * c->E) return fail(MOE_EINVAL, "moe_cache_slot_of: bad argument");
  *slot = c->lru.slot_of(key);
  return MOE_OK;
}

int moe_cache_resize(moe_cache_t* c, int S_new, moe_move_t* moves, int max_moves, int* n_moves) {
  if (!c || !n_moves || max_moves < 0 || (max_moves > 0 && !moves))
    return fail(MOE_EINVAL, "moe_cache_resize: null argument");
  if (S_new < 1) return fail(MOE_ECAPACITY, "moe_cache_resize: the cache needs at least one slot (S=%d)", S_new);
  std::vector<moe::Move> mv;
  moe::SharedLru next = c->lru;  // planned on a copy, so that a short move array changes nothing
  next.resize(S_new, mv);
  if ((int)mv.size() > max_moves)
    return fail(MOE_EINVAL, "moe_cache_resize: %d moves do not fit %d", (int)mv.size(), max_moves);
  c->lru = std::move(next);
  c->S = S_new;
  for (size_t i = 0; i < mv.size(); ++i) moves[i] = moe_move_t{mv[i].key, mv[i].from, mv[i].to};
  *n_moves = (int)mv.size();
  return MOE_OK;
}

int moe_cache_capacity(const moe_cache_t* c) { return c ? c->S : 0; }

int moe_cache_stats(const moe_cache_t* c, int64_t* hits, int64_t* misses) {
  if (!c || !hits || !misses) return fail(MOE_EINVAL, "moe_cache_stats: null pointer");
  *hits = c->lru.hits();
  *misses = c->lru.misses();
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Fills
// ---------------------------------------------------------------------------
}  // extern "C"

// The copies of cache_fill_async, ordered after every earlier reader on the
// compute stream (or, with war_after, after that event, which the caller
// recorded after every reader of the victim slots; with readers_done, after
// nothing: the caller has seen every reader of the victim slots complete);
// *done (the cache's event) marks their end on the fill stream, and the
// compute stream is not yet made to wait for it.
int cache_fill_enqueue(moe_cache_t* c, const moe_miss_t* misses, int n, const void* const* layer_pool,
                       size_t blob_stride, size_t blob_bytes, void* slot_base, size_t slot_stride, void* fill_stream,
                       void* compute_stream, hipEvent_t* done, hipEvent_t war_after = nullptr,
                       bool readers_done = false);

extern "C" {

int cache_fill_async(moe_cache_t* c, const moe_miss_t* misses, int n, const void* const* layer_pool,
                     size_t blob_stride, size_t blob_bytes, void* slot_base, size_t slot_stride, void* fill_stream,
                     void* compute_stream) {
  hipEvent_t done = nullptr;
  const int rc = cache_fill_enqueue(c, misses, n, layer_pool, blob_stride, blob_bytes, slot_base, slot_stride,
                                    fill_stream, compute_stream, &done);
  if (rc != MOE_OK || !done) return rc;
  hipError_t e = hipStreamWaitEvent(as_stream(compute_stream), done, 0);
  if (e == hipSuccess) return MOE_OK;
  for (int i = 0; i < n; ++i) (void)c->lru.invalidate(misses[i].key);  // no reader would wait for the copies
  return hip_fail(e, "cache_fill_async: ordering before compute");
}

}  // extern "C"

int cache_fill_enqueue(moe_cache_t* c, const moe_miss_t* misses, int n, const void* const* layer_pool,
                       size_t blob_stride, size_t blob_bytes, void* slot_base, size_t slot_stride, void* fill_stream,
                       void* compute_stream, hipEvent_t* done, hipEvent_t war_after, bool readers_done) {
  *done = nullptr;
  if (!c || n < 0 || (n > 0 && !misses)) return fail(MOE_EINVAL, "cache_fill_async: bad argument");
  if (n == 0) return MOE_OK;
  // Whatever fails below, no key of the batch may stay mapped to a slot that
  // its copy has not reached (or that no reader is ordered after).
  const auto drop_from = [&](int i0, int rc) {
    for (int j = i0; j < n; ++j)
      if (misses[j].key >= 0 && misses[j].key < c->L * c->E) (void)c->lru.invalidate(misses[j].key);
    return rc;
  };
  if (!layer_pool || !slot_base || blob_bytes > slot_stride || blob_bytes > blob_stride)
    return drop_from(0, fail(MOE_EINVAL, "cache_fill_async: bad argument"));
  for (int i = 0; i < n; ++i)
    if (misses[i].key < 0 || misses[i].key >= c->L * c->E || misses[i].slot < 0 || misses[i].slot >= c->S)
      return drop_from(0, fail(MOE_EINVAL, "cache_fill_async: miss %d has key %d slot %d out of range", i,
                               misses[i].key, misses[i].slot));
  hipStream_t fs = as_stream(fill_stream), cs = as_stream(compute_stream);
  hipError_t e = hipSuccess;
  if (!c->ev_war) e = hipEventCreateWithFlags(&c->ev_war, hipEventDisableTiming);
  if (e == hipSuccess && !c->ev_done) e = hipEventCreateWithFlags(&c->ev_done, hipEventDisableTiming);
  if (e != hipSuccess) return drop_from(0, hip_fail(e, "cache_fill_async: event create"));
  const bool split = fs != cs;
  if (split && !readers_done) {
    if (war_after) {
      e = hipStreamWaitEvent(fs, war_after, 0);
    } else {
      e = hipEventRecord(c->ev_war, cs);
      if (e == hipSuccess) e = hipStreamWaitEvent(fs, c->ev_war, 0);
    }
    if (e != hipSuccess) return drop_from(0, hip_fail(e, "cache_fill_async: ordering after compute"));
  }
  char* dst = static_cast<char*>(slot_base);
  std::vector<int32_t> keys(n);
  for (int i = 0; i < n; ++i) keys[i] = misses[i].key;
  int rc = MOE_OK;
  const auto copy = [&](int i) {
    const int layer = misses[i].key / c->E, ex = misses[i].key % c->E;
    const char* src = static_cast<const char*>(layer_pool[layer]);
    if (!src) {
      rc = fail(MOE_EINVAL, "cache_fill_async: no pool address for layer %d", layer);
      return false;
    }
    char* slot = dst + (size_t)misses[i].slot * slot_stride;
    if (c->poison) {  // debug: a read of the slot before the copy lands sees NaN
      e = moe::launch_poison(slot, blob_bytes, fs);
      if (e != hipSuccess) {
        rc = hip_fail(e, "cache_fill_async: poison");
        return false;
      }
    }
    e = hipMemcpyAsync(slot, src + (size_t)ex * blob_stride, blob_bytes, hipMemcpyHostToDevice, fs);
    if (e != hipSuccess) {
      rc = hip_fail(e, "cache_fill_async: copy");
      return false;
    }
    return true;
  };
  // A miss whose copy is not issued, and every later one, is dropped here;
  // the copies issued before it keep their keys.
  const int issued = moe::issue_fills(c->lru, keys.data(), n, copy);
  if (split) {
    e = hipEventRecord(c->ev_done, fs);
    if (e != hipSuccess) return drop_from(0, issued < n ? rc : hip_fail(e, "cache_fill_async: completion event"));
    if (issued < n) {
      // the call fails, so the caller will not wait: order later readers of
      // the issued copies after them here
      e = hipStreamWaitEvent(cs, c->ev_done, 0);
      return e == hipSuccess ? rc : drop_from(0, rc);
    }
    *done = c->ev_done;
  }
  return rc;
}

extern "C" {

// ---------------------------------------------------------------------------
// Expert FFN
// ---------------------------------------------------------------------------
size_t moe_ffn_workspace_size(int rows_total, int H, int I, int wfmt) {
  if (rows_total < 0 || !shape_ok(wfmt, H, I)) return 0;
  // h: one row of I per routed row, plus one 16-row tile of slack for the
  // prefill GEMM's tiled h layout
  const size_t hb = moe::align_up((size_t)(rows_total + 16) * I * (wfmt == MOE_W_F32 ? 4 : 2), 256);
  return hb + 4 * moe::kTableBytes + 256;
}

int moe_ffn(const void* x, int dtype, const int32_t* perm_src, const moe_work_t* work, int n_work,
            const void* slot_base, size_t slot_stride, int wfmt, int H, int I, float* y_perm, void* workspace,
            size_t ws_bytes, int mode, void* stream) {
  if (!shape_ok(wfmt, H, I)) return fail(MOE_EINVAL, "moe_ffn: unsupported format/shape %d %dx%d", wfmt, H, I);
  if ((wfmt == MOE_W_F32) != (dtype == MOE_DT_F32) || (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16))
    return fail(MOE_EINVAL, "moe_ffn: activation dtype %d does not match weight format %d", dtype, wfmt);
  if (n_work < 0 || (n_work > 0 && (!work || !x || !perm_src || !slot_base || !y_perm || !workspace)))
    return fail(MOE_EINVAL, "moe_ffn: null pointer or negative count");
  if (mode < MOE_FFN_AUTO || mode > MOE_FFN_PREFILL) return fail(MOE_EINVAL, "moe_ffn: bad mode %d", mode);
  if (n_work == 0) return MOE_OK;
  const size_t blob = moe::blob_layout(wfmt, H, I).bytes;
  if (slot_stride < blob) return fail(MOE_EINVAL, "moe_ffn: slot_stride %zu < blob size %zu", slot_stride, blob);
  int rows_total = 0, max_rows = 0;
  for (int i = 0; i < n_work; ++i) {
    const moe_work_t& w = work[i];
    if (w.rows < 0 || w.row_begin < 0 || w.slot < 0)
      return fail(MOE_EINVAL, "moe_ffn: work item %d has negative field", i);
    rows_total = std::max(rows_total, w.row_begin + w.rows);
    max_rows = std::max(max_rows, w.rows);
  }
  if (ws_bytes < moe_ffn_workspace_size(rows_total, H, I, wfmt))
    return fail(MOE_EINVAL, "moe_ffn: workspace too small for %d rows", rows_total);
  bool prefill = false;
  const bool gemm_ok = wfmt == MOE_W_MXFP4 ? moe::prefill_mxfp4_supported(H, I) : moe::prefill_supported(wfmt, H, I);
  if (mode == MOE_FFN_PREFILL) {
    if (!gemm_ok)
      return fail(MOE_EINVAL,
                  "moe_ffn: prefill GEMM needs bf16 weights with H %% 128 == 0 and I %% 64 == 0, or MXFP4 weights "
                  "with H %% 256 == 0");
    prefill = true;
  } else if (mode == MOE_FFN_AUTO) {
    prefill = max_rows > 32 && gemm_ok;
  }
  char* ws = static_cast<char*>(workspace);
  void* hbuf = ws;
  void* tables = ws + moe::align_up((size_t)(rows_total + 16) * I * (wfmt == MOE_W_F32 ? 4 : 2), 256);
  hipStream_t s = as_stream(stream);
  if (prefill && wfmt == MOE_W_MXFP4) {
    std::vector<int4> items;
    items.reserve(n_work);
    for (int i = 0; i < n_work; ++i)
      if (work[i].rows > 0) items.push_back(make_int4(work[i].slot, work[i].row_begin, work[i].rows, work[i].expert));
    for (size_t base = 0; base < items.size(); base += moe::kTableItems) {
      const int n = (int)std::min(items.size() - base, (size_t)moe::kTableItems);
      hipError_t e = moe::launch_ffn_prefill_mxfp4(x, perm_src, items.data() + base, n,
                                                   static_cast<const char*>(slot_base), slot_stride, H, I, hbuf,
                                                   y_perm, tables, s);
      if (e != hipSuccess) return hip_fail(e, "moe_ffn launch");
    }
    return MOE_OK;
  }
  if (prefill && moe::gemm2_supported(2 * I, H) && moe::gemm2_supported(H, I)) {
    // large-tile GEMM: the whole work list per launch, from a device table
    std::vector<int4> items;
    items.reserve(n_work);
    for (int i = 0; i < n_work; ++i)
      if (work[i].rows > 0) items.push_back(make_int4(work[i].slot, work[i].row_begin, work[i].rows, work[i].expert));
    for (size_t base = 0; base < items.size(); base += moe::kTableItems) {
      const int n = (int)std::min(items.size() - base, (size_t)moe::kTableItems);
      hipError_t e = moe::launch_ffn_prefill2(x, perm_src, items.data() + base, n, static_cast<const char*>(slot_base),
                                              slot_stride, H, I, hbuf, y_perm, tables, s);
      if (e != hipSuccess) return hip_fail(e, "moe_ffn launch");
    }
    return MOE_OK;
  }
  moe::WorkArgs wa;
  for (int base = 0; base < n_work; base += moe::kMaxItems) {
    std::memset(&wa, 0, sizeof wa);
    int n = 0;
    for (int i = base; i < n_work && n < moe::kMaxItems; ++i) {
      if (work[i].rows == 0) continue;
      wa.item[n++] = make_int4(work[i].slot, work[i].row_begin, work[i].rows, work[i].expert);
    }
    wa.n = n;
    if (n == 0) continue;
    hipError_t e = prefill ? moe::launch_ffn_prefill(x, perm_src, wa, static_cast<const char*>(slot_base), slot_stride,
                                                     H, I, hbuf, y_perm, s)
                           : moe::launch_ffn_decode(wfmt, x, perm_src, wa, static_cast<const char*>(slot_base),
                                                    slot_stride, H, I, hbuf, y_perm, s);
    if (e != hipSuccess) return hip_fail(e, "moe_ffn launch");
  }
  return MOE_OK;
}

int moe_ffn_grouped(const void* x, int dtype, const int32_t* perm_src, const int32_t* counts, const int32_t* offsets,
                    const int32_t* slot_of, int E, int n_slots, int rows_max, const void* slot_base,
                    size_t slot_stride, int wfmt, int H, int I, float* y_perm, void* workspace, size_t ws_bytes,
                    void* stream) {
  if (!moe::grouped_supported(wfmt, H, I))
    return fail(MOE_EINVAL,
                "moe_ffn_grouped: needs bf16 weights with H and 2I multiples of 256 and I of 32, or MXFP4 weights "
                "with H %% 256 == 0 and I %% 128 == 0 (got format %d, %dx%d)",
                wfmt, H, I);
  if (dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "moe_ffn_grouped: activations must be bf16");
  if (E < 1 || E > 1024 || n_slots < 1 || rows_max < 0)
    return fail(MOE_EINVAL, "moe_ffn_grouped: bad sizes E=%d n_slots=%d rows_max=%d", E, n_slots, rows_max);
  if (!x || !perm_src || !counts || !offsets || !slot_base || !y_perm || !workspace)
    return fail(MOE_EINVAL, "moe_ffn_grouped: null pointer argument");
  const size_t blob = moe::blob_layout(wfmt, H, I).bytes;
  if (slot_stride < blob) return fail(MOE_EINVAL, "moe_ffn_grouped: slot_stride %zu < blob size %zu", slot_stride, blob);
  if (ws_bytes < moe_ffn_workspace_size(rows_max, H, I, wfmt))
    return fail(MOE_EINVAL, "moe_ffn_grouped: workspace too small for %d rows", rows_max);
  if (rows_max == 0) return MOE_OK;
  char* ws = static_cast<char*>(workspace);
  const size_t hb = moe::align_up((size_t)(rows_max + 16) * I * 2, 256);
  hipError_t e = moe::launch_ffn_grouped(wfmt, x, perm_src, counts, offsets, slot_of, E, n_slots, rows_max,
                                         static_cast<const char*>(slot_base), slot_stride, H, I, ws, y_perm, ws + hb,
                                         as_stream(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_ffn_grouped launch");
}

// ---------------------------------------------------------------------------
// Combine
// ---------------------------------------------------------------------------
int moe_combine(const float* y_perm, const int32_t* perm_pos, const float* topk_w, int T, int k, int H, void* out,
                int out_dtype, void* stream) {
  if (T < 0 || k < 1 || H < 1 || (out_dtype != MOE_DT_F32 && out_dtype != MOE_DT_BF16))
    return fail(MOE_EINVAL, "moe_combine: bad sizes or dtype");
  if (T > 0 && (!y_perm || !perm_pos || !topk_w || !out)) return fail(MOE_EINVAL, "moe_combine: null pointer");
  hipError_t e = moe::launch_combine(y_perm, perm_pos, topk_w, T, k, H, out, out_dtype == MOE_DT_BF16,
                                     as_stream(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine launch");
}

// ---------------------------------------------------------------------------
// Prefill double buffering
// ---------------------------------------------------------------------------
static void pipe_release(moe_pipe_t* p) {
  for (auto v : {&p->copied, &p->started, &p->done})
    for (hipEvent_t ev : *v)
      if (ev) (void)hipEventDestroy(ev);
  for (void* b : p->buf)
    if (b) (void)hipFree(b);
  if (p->copy) (void)hipStreamDestroy(p->copy);
  delete p;
}

moe_pipe_t* moe_pipe_create(const void* const* layer_src, size_t layer_bytes, int n_layers, int* status) {
  bool ok = layer_src && n_layers > 0 && layer_bytes > 0;
  for (int l = 0; ok && l < n_layers; ++l) ok = layer_src[l] != nullptr;
  if (!ok) {
    if (status) *status = fail(MOE_EINVAL, "moe_pipe_create: bad argument");
    return nullptr;
  }
  moe_pipe_t* p = new (std::nothrow) moe_pipe();
  if (!p) {
    if (status) *status = fail(MOE_ENOMEM, "moe_pipe_create: out of host memory");
    return nullptr;
  }
  for (int l = 0; l < n_layers; ++l) p->src.push_back(static_cast<const char*>(layer_src[l]));
  p->bytes = layer_bytes;
  p->L = n_layers;
  p->copied.assign(n_layers, nullptr);
  p->started.assign(n_layers, nullptr);
  p->done.assign(n_layers, nullptr);
  hipError_t e = hipSuccess;
  for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipMalloc(&p->buf[i], layer_bytes);
  if (e != hipSuccess) {
    pipe_release(p);
    if (status) *status = fail(MOE_ENOMEM, "moe_pipe_create: device buffers: %s", hipGetErrorString(e));
    return nullptr;
  }
  e = hipStreamCreateWithFlags(&p->copy, hipStreamNonBlocking);
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    e = hipEventCreate(&p->copied[l]);
    if (e == hipSuccess) e = hipEventCreate(&p->started[l]);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->done[l], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    pipe_release(p);
    if (status) *status = fail(MOE_EHIP, "moe_pipe_create: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (status) *status = MOE_OK;
  return p;
}

int moe_pipe_destroy(moe_pipe_t* p) {
  if (!p) return MOE_OK;
  if (p->copy) (void)hipStreamSynchronize(p->copy);
  pipe_release(p);
  return MOE_OK;
}

static hipError_t pipe_start_copy(moe_pipe_t* p, int l) {
  hipError_t e = hipSuccess;
  if (l >= 2) e = hipStreamWaitEvent(p->copy, p->done[l - 2], 0);  // buffer l%2 was last read by layer l-2
  if (e == hipSuccess) e = hipEventRecord(p->started[l], p->copy);
  if (e == hipSuccess)
    e = hipMemcpyAsync(p->buf[l & 1], p->src[l], p->bytes, hipMemcpyHostToDevice, p->copy);
  if (e == hipSuccess) e = hipEventRecord(p->copied[l], p->copy);
  if (e == hipSuccess) p->next_copy = l + 1;
  return e;
}

int moe_pipe_begin_layer(moe_pipe_t* p, int layer, void* compute_stream, void** buffer) {
  if (!p || !buffer) return fail(MOE_EINVAL, "moe_pipe_begin_layer: null pointer");
  if (layer != p->next_begin || layer >= p->L)
    return fail(MOE_ESTATE, "moe_pipe_begin_layer: expected layer %d, got %d", p->next_begin, layer);
  if (p->next_end != layer)  // the copy of layer+1 must be ordered after layer-1's compute
    return fail(MOE_ESTATE, "moe_pipe_begin_layer: layer %d has not ended", layer - 1);
  hipError_t e = hipSuccess;
  if (p->next_copy == layer) e = pipe_start_copy(p, layer);
  hipStream_t cs = as_stream(compute_stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(cs, p->copied[layer], 0);
  if (e == hipSuccess && layer + 1 < p->L && p->next_copy == layer + 1) e = pipe_start_copy(p, layer + 1);
  if (e != hipSuccess) return hip_fail(e, "moe_pipe_begin_layer");
  *buffer = p->buf[layer & 1];
  p->next_begin = layer + 1;
  return MOE_OK;
}

int moe_pipe_end_layer(moe_pipe_t* p, int layer, void* compute_stream) {
  if (!p || layer != p->next_end || layer >= p->next_begin)
    return fail(MOE_ESTATE, "moe_pipe_end_layer: layer %d has not begun or already ended", layer);
  hipError_t e = hipEventRecord(p->done[layer], as_stream(compute_stream));
  if (e != hipSuccess) return hip_fail(e, "moe_pipe_end_layer");
  p->next_end = layer + 1;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Prefill layer: routing, grouped FFN over the device work list, combine
// ---------------------------------------------------------------------------
int moe_prefill_layer(const void* x, int dtype, const void* Wr, const float* bias, int T, int H, int E, int k, int I,
                      int wfmt, const void* layer_base, size_t blob_stride, const moe_decoder_buffers_t* b, void* out,
                      int out_dtype, void* stream) {
  if (!b) return fail(MOE_EINVAL, "moe_prefill_layer: null buffers");
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || (long long)T * k > (1ll << 30))
    return fail(MOE_EINVAL, "moe_prefill_layer: bad sizes T=%d H=%d E=%d k=%d", T, H, E, k);
  if (!moe::grouped_supported(wfmt, H, I) || dtype != MOE_DT_BF16)
    return fail(MOE_EINVAL, "moe_prefill_layer: needs bf16 activations and bf16 or MXFP4 experts of a shape the "
                            "grouped GEMM takes (format %d, %dx%d)", wfmt, H, I);
  if (T > 0 && (!out || !b->y_perm || !layer_base)) return fail(MOE_EINVAL, "moe_prefill_layer: null pointer");
  if (out_dtype != MOE_DT_F32 && out_dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "moe_prefill_layer: bad out dtype");
  int rc = moe_route(x, dtype, Wr, bias, T, H, E, k, b->topk_idx, b->topk_w, b->logits, b->counts, b->offsets,
                     b->perm_src, b->perm_pos, b->route_ws, b->route_ws_bytes, stream);
  if (rc != MOE_OK || T == 0) return rc;
  rc = moe_ffn_grouped(x, dtype, b->perm_src, b->counts, b->offsets, nullptr, E, E, T * k, layer_base, blob_stride,
                       wfmt, H, I, b->y_perm, b->ffn_ws, b->ffn_ws_bytes, stream);
  if (rc != MOE_OK) return rc;
  return moe_combine(b->y_perm, b->perm_pos, b->topk_w, T, k, H, out, out_dtype, stream);
}

int moe_clock_record(unsigned long long* sums) {
  moe::set_clock_sums(sums);
  return MOE_OK;
}

int moe_pipe_copy_ms(moe_pipe_t* p, int layer, float* ms) {
  if (!p || !ms || layer < 0 || layer >= p->next_copy) return fail(MOE_EINVAL, "moe_pipe_copy_ms: bad layer");
  hipError_t e = hipEventElapsedTime(ms, p->started[layer], p->copied[layer]);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pipe_copy_ms");
}

}  // extern "C"
