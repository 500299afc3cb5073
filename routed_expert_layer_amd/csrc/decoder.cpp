// Native decode layer-step: the calls of the C ABI sequenced in C++ so that
// one layer-step costs one host round trip (the per-expert counts) and no
// interpreter overhead.
//
// Page "FreeToken-rtx-4090", phase table row "Decode": the bottleneck is
// expert cache misses and the mechanism is the shared LRU cache; the
// component table's "PCIe link" row: only the missing experts move.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_kernels.hpp"

extern "C" const char* moe_last_error(void);
int moe_cache_layers(const moe_cache_t* c, int* n_layers);
int moe_cache_experts(const moe_cache_t* c);
bool moe_cache_splits(const moe_cache_t* c);
uint64_t moe_cache_edits(const moe_cache_t* c);
int cache_fill_enqueue(moe_cache_t* c, const moe_miss_t* misses, int n, const void* const* layer_pool,
                       size_t blob_stride, size_t blob_bytes, void* slot_base, size_t slot_stride, void* fill_stream,
                       void* compute_stream, hipEvent_t* done, hipEvent_t war_after, bool readers_done);

namespace {
// Errors go to the library's per-thread message (moe_last_error).
template <typename... A>
int dfail(int code, const char* fmt, A... a) {
  return moe::set_error(code, fmt, a...);
}
}  // namespace

struct moe_decoder {
  moe_cache_t* cache;
  int Tmax, H, I, E, k, dtype, wfmt;
  std::vector<const void*> layer_pool;
  size_t blob_stride, blob_bytes;
  void* slot_base;
  size_t slot_stride;
  moe_decoder_buffers_t b;
  int32_t* counts_host = nullptr;  // pinned, host address
  std::vector<int32_t> counts;     // this step's counts, read from counts_host
  int32_t* counts_dev = nullptr;   // the same memory as seen by kernels
  hipStream_t fill = nullptr;
  hipEvent_t ev_counts = nullptr;
  int32_t route_seq = 0;  // number of the last routing launch (1..65535, carried by each count word)
  std::vector<int32_t> experts, work_e, work_slot, work_wave;
  std::vector<moe_miss_t> misses, wave_misses;
  std::vector<moe_work_t> work;
  std::vector<int32_t> offs;
  int prof_every = 0;     // bracket every prof_every-th FFN call with events (0: off)
  int64_t prof_calls = 0;  // FFN calls since profiling was enabled
  std::vector<hipEvent_t> ev_begin, ev_end;
  std::vector<double> ev_bytes;
  size_t ev_used = 0;
  int64_t fills = 0;
  // CPU execution of misses (when the cache splits them): pinned copies of
  // the step's activations and token order, and the CPU results on their way
  // into y_perm
  uint16_t* x_host = nullptr;
  int32_t* perm_host = nullptr;
  float* y_host = nullptr;
  std::vector<uint16_t> xg;
  int64_t cpu_runs = 0;
  // Decode batches (T <= 16): the hits' FFN is enqueued right after the
  // routing, from a copy of the cache's slot table kept on the GPU, instead
  // of after the host's resolve; the host's round trip then overlaps it.
  int32_t* slot_of_dev = nullptr;  // [L*E], the copy the kernels read
  std::vector<int32_t> slot_of;    // what the GPU copy holds (after the updates enqueued so far)
  uint64_t slot_of_edits = ~0ull;  // the cache's edit count the copy matches (~0: never uploaded)
  moe::SlotUpdates pending{};      // updates for the GPU copy, applied by the next routing launch
  int32_t* hit_n = nullptr;        // device: number of resident-expert items
  int4* hit_items = nullptr;       // device: [E] items {slot, first row, rows, expert}
  uint64_t* ffn_flags = nullptr;   // device: hand-off flags of the one-launch FFN (zeroed at creation)
  uint64_t ffn_seq = 0;            // the last call's flag value
  int n_layers = 0;
};

extern "C" {

static void decoder_release(moe_decoder_t* d) {
  if (d->counts_host) (void)hipHostFree(d->counts_host);
  if (d->x_host) (void)hipHostFree(d->x_host);
  if (d->perm_host) (void)hipHostFree(d->perm_host);
  if (d->y_host) (void)hipHostFree(d->y_host);
  if (d->fill) (void)hipStreamDestroy(d->fill);
  if (d->ev_counts) (void)hipEventDestroy(d->ev_counts);
  if (d->slot_of_dev) (void)hipFree(d->slot_of_dev);
  if (d->hit_n) (void)hipFree(d->hit_n);
  if (d->ffn_flags) (void)hipFree(d->ffn_flags);
  for (hipEvent_t e : d->ev_begin) (void)hipEventDestroy(e);
  for (hipEvent_t e : d->ev_end) (void)hipEventDestroy(e);
  delete d;
}

moe_decoder_t* moe_decoder_create(moe_cache_t* cache, int T_max, int H, int I, int E, int k, int dtype, int wfmt,
                                  const void* const* layer_pool, size_t blob_stride, void* slot_base,
                                  size_t slot_stride, const moe_decoder_buffers_t* buffers, int* status) {
  auto bad = [&](int code, const char* msg) -> moe_decoder_t* {
    if (status) *status = dfail(code, "moe_decoder_create: %s", msg);
    return nullptr;
  };
  if (!cache || !layer_pool || !slot_base || !buffers) return bad(MOE_EINVAL, "null argument");
  if (T_max < 1 || H < 1 || I < 1 || E < 1 || E > 1024 || k < 1 || k > 16 || k > E || H % 8 != 0)
    return bad(MOE_EINVAL, "bad sizes");
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return bad(MOE_EINVAL, "bad activation dtype");
  const size_t blob = moe_expert_bytes(wfmt, H, I);
  if (blob == 0) return bad(MOE_EINVAL, "unsupported weight format or shape");
  if (blob_stride < blob || slot_stride < blob) return bad(MOE_EINVAL, "stride smaller than an expert blob");
  const moe_decoder_buffers_t& b = *buffers;
  if (!b.topk_idx || !b.topk_w || !b.counts || !b.offsets || !b.perm_src || !b.perm_pos || !b.y_perm ||
      !b.route_ws || !b.ffn_ws)
    return bad(MOE_EINVAL, "null device buffer");
  if (b.route_ws_bytes < moe_route_workspace_size(T_max, H, E, k)) return bad(MOE_EINVAL, "route workspace too small");
  if (b.ffn_ws_bytes < moe_ffn_workspace_size(T_max * k, H, I, wfmt)) return bad(MOE_EINVAL, "FFN workspace too small");
  moe_decoder_t* d = new (std::nothrow) moe_decoder();
  if (!d) return bad(MOE_ENOMEM, "out of host memory");
  d->cache = cache;
  d->Tmax = T_max; d->H = H; d->I = I; d->E = E; d->k = k; d->dtype = dtype; d->wfmt = wfmt;
  int n_layers = 0;
  if (moe_cache_layers(cache, &n_layers) != MOE_OK || moe_cache_experts(cache) != E) {
    delete d;
    return bad(MOE_EINVAL, "cache does not match E");
  }
  for (int l = 0; l < n_layers; ++l) {
    if (!layer_pool[l]) {
      delete d;
      return bad(MOE_EINVAL, "null layer pool address");
    }
    d->layer_pool.push_back(layer_pool[l]);
  }
  d->blob_stride = blob_stride; d->blob_bytes = blob;
  d->slot_base = slot_base; d->slot_stride = slot_stride;
  d->b = b;
  // fine-grained (coherent) pinned memory that the routing kernels write directly
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&d->counts_host), sizeof(int32_t) * E,
                               hipHostMallocMapped | hipHostMallocCoherent);
  if (e == hipSuccess) std::memset(d->counts_host, 0, sizeof(int32_t) * E);
  d->counts.assign(E, 0);
  if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void**>(&d->counts_dev), d->counts_host, 0);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&d->fill, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&d->ev_counts, hipEventDisableTiming);
  d->n_layers = n_layers;
  d->slot_of.assign((size_t)n_layers * E, -1);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&d->slot_of_dev), sizeof(int32_t) * d->slot_of.size());
  // hit_n, then the items 16-byte aligned
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&d->hit_n), 16 + sizeof(int4) * E);
  if (e == hipSuccess) d->hit_items = reinterpret_cast<int4*>(reinterpret_cast<char*>(d->hit_n) + 16);
  if (e == hipSuccess && moe::ffn_fused_ok(wfmt, H, I)) {
    const size_t fb = sizeof(uint64_t) * moe::ffn_fused_flags(E, I);
    e = hipMalloc(reinterpret_cast<void**>(&d->ffn_flags), fb);
    if (e == hipSuccess) e = hipMemset(d->ffn_flags, 0, fb);
  }
  if (e != hipSuccess) {
    decoder_release(d);
    if (status) *status = dfail(MOE_EHIP, "moe_decoder_create: %s", hipGetErrorString(e));
    return nullptr;
  }
  d->experts.reserve(E);
  d->offs.resize(E + 1);
  if (status) *status = MOE_OK;
  return d;
}

int moe_decoder_destroy(moe_decoder_t* d) {
  if (!d) return MOE_OK;
  if (d->fill) (void)hipStreamSynchronize(d->fill);
  decoder_release(d);
  return MOE_OK;
}

static int record_ffn_event(moe_decoder_t* d, bool begin, hipStream_t s, double bytes) {
  if (begin) {
    if (d->ev_used == d->ev_begin.size()) {
      hipEvent_t a, c;
      if (hipEventCreate(&a) != hipSuccess) return MOE_EHIP;
      if (hipEventCreate(&c) != hipSuccess) {
        (void)hipEventDestroy(a);
        return MOE_EHIP;
      }
      d->ev_begin.push_back(a);
      d->ev_end.push_back(c);
      d->ev_bytes.push_back(0.0);
    }
    return hipEventRecord(d->ev_begin[d->ev_used], s) == hipSuccess ? MOE_OK : MOE_EHIP;
  }
  d->ev_bytes[d->ev_used] = bytes;
  hipError_t e = hipEventRecord(d->ev_end[d->ev_used], s);
  ++d->ev_used;
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Brings the GPU copy of the slot table in line with the cache when the cache
// was changed other than by a resolve (invalidation, resize) or has never
// been copied: a full upload, after the stream has drained so that no queued
// kernel still reads the copy.
static int sync_slot_table(moe_decoder_t* d, hipStream_t s) {
  const uint64_t ed = moe_cache_edits(d->cache);
  if (ed == d->slot_of_edits) return MOE_OK;
  for (size_t key = 0; key < d->slot_of.size(); ++key) {
    int sl = -1;
    (void)moe_cache_slot_of(d->cache, (int)key, &sl);
    d->slot_of[key] = sl;
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess)
    e = hipMemcpy(d->slot_of_dev, d->slot_of.data(), sizeof(int32_t) * d->slot_of.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return dfail(MOE_EHIP, "moe_decoder_step: slot table upload: %s", hipGetErrorString(e));
  d->slot_of_edits = ed;
  d->pending.n = 0;  // the upload holds them
  return MOE_OK;
}

// After the resolve: the experts the GPU listed as resident must be exactly
// the resolve's hits, in the same slots; then the copy takes this step's
// fills (the miss's key in its slot, the victim's key out): up to
// kSlotUpdatesMax of them ride with the next routing launch, the rest go now
// in their own launches on the stream.
static int update_slot_table(moe_decoder_t* d, int layer, int n, int nm, hipStream_t s) {
  for (int i = 0; i < n; ++i) {
    const int key = layer * d->E + d->work_e[i];
    bool miss = d->work_slot[i] < 0;
    for (int j = 0; j < nm && !miss; ++j) miss = d->misses[j].key == key;
    const int32_t copy = d->slot_of[key];
    if (miss ? copy >= 0 : copy != d->work_slot[i]) {
      d->slot_of_edits = ~0ull;  // upload the whole table before the next step
      return dfail(MOE_EHIP, "moe_decoder_step: the GPU copy of the slot table disagrees with the cache at key %d",
                   key);
    }
  }
  std::vector<int32_t> touched;
  for (int j = 0; j < nm; ++j) {
    const moe_miss_t& m = d->misses[j];
    if (m.victim >= 0) {
      d->slot_of[m.victim] = -1;
      touched.push_back(m.victim);
    }
    d->slot_of[m.key] = m.slot;
    touched.push_back(m.key);
  }
  std::sort(touched.begin(), touched.end());
  touched.erase(std::unique(touched.begin(), touched.end()), touched.end());
  d->pending.n = (int)std::min<size_t>(moe::kSlotUpdatesMax, touched.size());
  for (int i = 0; i < d->pending.n; ++i) {
    d->pending.key[i] = touched[i];
    d->pending.slot[i] = d->slot_of[touched[i]];
  }
  for (size_t i0 = moe::kSlotUpdatesMax; i0 < touched.size(); i0 += moe::kSlotUpdatesMax) {
    moe::SlotUpdates u;
    u.n = (int)std::min<size_t>(moe::kSlotUpdatesMax, touched.size() - i0);
    for (int i = 0; i < u.n; ++i) {
      u.key[i] = touched[i0 + i];
      u.slot[i] = d->slot_of[touched[i0 + i]];
    }
    const hipError_t e = moe::launch_slot_updates(d->slot_of_dev, u, s);
    if (e != hipSuccess) {
      d->slot_of_edits = ~0ull;
      return dfail(MOE_EHIP, "moe_decoder_step: slot table update: %s", hipGetErrorString(e));
    }
  }
  return MOE_OK;
}

int moe_decoder_step(moe_decoder_t* d, int step, int layer, const void* x, int T, const void* Wr, const float* bias,
                     void* out, int out_dtype, void* stream, int* n_miss) {
  if (!d || !x || !Wr || !out) return dfail(MOE_EINVAL, "moe_decoder_step: null argument");
  if (T < 1 || T > d->Tmax) return dfail(MOE_EINVAL, "moe_decoder_step: T=%d outside [1, %d]", T, d->Tmax);
  if (out_dtype != MOE_DT_F32 && out_dtype != MOE_DT_BF16)
    return dfail(MOE_EINVAL, "moe_decoder_step: out_dtype %d is neither MOE_DT_F32 nor MOE_DT_BF16", out_dtype);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const moe_decoder_buffers_t& b = d->b;
  // decode batches run the resident experts' FFN ahead of the resolve (below)
  const bool early_hits = moe::route_small_path(T, d->E);
  if (early_hits) {
    const int rc0 = sync_slot_table(d, s);
    if (rc0 != MOE_OK) return rc0;
  }
  // routing; the kernels also store the per-expert counts straight into the
  // host-mapped pinned buffer: the one device -> host transfer of the step
  const int32_t seq = d->route_seq = d->route_seq >= 65535 ? 1 : d->route_seq + 1;
  const bool tagged = moe::route_small_path(T, d->E);
  moe::ResidentList res{};
  if (early_hits) {
    res.slot_of = d->slot_of_dev;
    res.layer = layer;
    res.n_out = d->hit_n;
    res.items = d->hit_items;
    res.updates = d->pending;
  }
  hipError_t e = moe::launch_route(x, d->dtype == MOE_DT_BF16, Wr, bias, T, d->H, d->E, d->k, b.topk_idx, b.topk_w,
                                   b.logits, b.counts, b.offsets, b.perm_src, b.perm_pos, b.route_ws, s,
                                   d->counts_dev, seq, early_hits ? &res : nullptr);
  if (e == hipSuccess) d->pending.n = 0;
  const bool split = moe_cache_splits(d->cache);
  if (split && e == hipSuccess) {
    // misses may run on the CPU: it needs this step's activations and token order
    if (d->dtype != MOE_DT_BF16 || d->wfmt == MOE_W_F32)
      return dfail(MOE_EINVAL,
                   "moe_decoder_step: CPU execution of misses needs bf16 activations and bf16, int4 or MXFP4 weights");
    if (!d->x_host) {
      e = hipHostMalloc(reinterpret_cast<void**>(&d->x_host), sizeof(uint16_t) * d->Tmax * d->H, hipHostMallocDefault);
      if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&d->perm_host), sizeof(int32_t) * d->Tmax * d->k,
                          hipHostMallocDefault);
      if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&d->y_host), sizeof(float) * d->Tmax * d->k * d->H,
                          hipHostMallocDefault);
      d->xg.resize((size_t)d->Tmax * d->H);
    }
    if (e == hipSuccess)
      e = hipMemcpyAsync(d->x_host, x, sizeof(uint16_t) * T * d->H, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(d->perm_host, b.perm_src, sizeof(int32_t) * T * d->k, hipMemcpyDeviceToHost, s);
  }
  // The counts event: the host waits on it for batches whose counts are not tagged and when misses run on the
  // CPU. For tagged decode batches with the early hits it is not recorded (every event between two kernels
  // costs the GPU ~1.5 us): the tagged counts show the routing done, and with it every earlier reader of a slot
  // (the stream runs in order), so the first wave's fills need no ordering at all; a failed launch is seen by
  // querying the stream.
  const bool counts_event = !(early_hits && tagged && !split);
  if (e == hipSuccess && counts_event) e = hipEventRecord(d->ev_counts, s);
  if (e != hipSuccess) return dfail(MOE_EHIP, "moe_decoder_step: routing: %s", hipGetErrorString(e));
  // The experts the GPU copy of the slot table shows as resident are the coming resolve's hits: the routing
  // kernel lists them and their FFN runs right after the routing, so it overlaps the counts' trip to the host,
  // the resolve and the fills' set-up instead of following them. The first wave's fills wait only for the work
  // before this FFN (their victims are never this step's hits); later waves' fills wait for everything before.
  bool prof_open = false;
  // bf16 decode steps of few experts: the resident experts' down projection also forms the step's output when
  // no expert is missing, and the combine launch is then left out
  const bool fused = early_hits && moe::ffn_combine_ok(d->wfmt, d->H, d->I, std::min(d->E, d->k * T), T, d->k);
  if (early_hits) {
    // ev_counts, when recorded (above, before this FFN), also orders the first wave's fills
    // profiled calls: every prof_every-th FFN of a layer-step whose experts were all resident; whether this
    // step is one is known after the resolve, so the events go out when the next such call is due
    if (d->prof_every > 0 && d->prof_calls % d->prof_every == 0) {
      if (record_ffn_event(d, true, s, 0) != MOE_OK) return dfail(MOE_EHIP, "moe_decoder_step: profiling event");
      prof_open = true;
    }
    if (e == hipSuccess && fused)
      e = moe::launch_ffn_decode_combine(x, b.perm_src, d->hit_n, d->hit_items, std::min(d->E, d->k * T), T,
                                         static_cast<const char*>(d->slot_base), d->slot_stride, d->H, d->I, b.ffn_ws,
                                         b.y_perm, d->hit_n + 1, b.perm_pos, b.topk_w, d->k, out,
                                         out_dtype == MOE_DT_BF16, s);
    else if (e == hipSuccess && d->ffn_flags != nullptr) {
      ++d->ffn_seq;
      e = moe::launch_ffn_decode_fused(d->wfmt, x, b.perm_src, d->hit_n, d->hit_items, std::min(d->E, d->k * T),
                                       static_cast<const char*>(d->slot_base), d->slot_stride, d->H, d->I, b.ffn_ws,
                                       b.y_perm, d->ffn_flags, d->ffn_seq, s);
    } else if (e == hipSuccess)
      e = moe::launch_ffn_decode_dev(d->wfmt, x, b.perm_src, d->hit_n, d->hit_items, std::min(d->E, d->k * T), T,
                                     static_cast<const char*>(d->slot_base), d->slot_stride, d->H, d->I, b.ffn_ws,
                                     b.y_perm, s);
    if (e == hipSuccess && prof_open) e = hipEventRecord(d->ev_end[d->ev_used], s);
    if (e != hipSuccess)
      return dfail(MOE_EHIP, "moe_decoder_step: resident experts' FFN: %s", hipGetErrorString(e));
  }
  int rc;
  bool all_resident = false;
  if (tagged && !split) {
    // decode batches: every count word carries this step's number, so the counts are complete once all of
    // them show it (the event is polled too, so a failed launch still ends the wait)
    for (unsigned spin = 1;; ++spin) {
      int e_ok = 0;
      for (int i = 0; i < d->E; ++i)
        e_ok += ((uint32_t)__atomic_load_n(d->counts_host + i, __ATOMIC_ACQUIRE) >> 16) == (uint32_t)seq;
      if (e_ok == d->E) break;
      // without the event, the stream is queried only after ~2^20 polls (far longer than a routing launch
      // takes): querying it meanwhile slows the step
      if ((spin & 63u) == 0 && (counts_event || spin >= (1u << 20))) {
        e = counts_event ? hipEventQuery(d->ev_counts) : hipStreamQuery(s);
        if (e != hipErrorNotReady) break;
        e = hipSuccess;
      }
    }
  } else {
    // larger batches, or misses on the CPU, which also need the activations and token order copied after
    // the routing: the event
    while ((e = hipEventQuery(d->ev_counts)) == hipErrorNotReady) {
    }
  }
  if (e != hipSuccess) return dfail(MOE_EHIP, "moe_decoder_step: counts wait: %s", hipGetErrorString(e));
  for (int i = 0; i < d->E; ++i) {
    const uint32_t w = (uint32_t)__atomic_load_n(d->counts_host + i, __ATOMIC_ACQUIRE);
    if (tagged && (w >> 16) != (uint32_t)seq)
      return dfail(MOE_EHIP, "moe_decoder_step: routing counts of step %d missing for expert %d", step, i);
    d->counts[i] = tagged ? (int32_t)(w & 0xFFFFu) : (int32_t)w;
  }
  d->experts.clear();
  int run = 0;
  for (int i = 0; i < d->E; ++i) {
    d->offs[i] = run;
    run += d->counts[i];
    if (d->counts[i] > 0) d->experts.push_back(i);
  }
  d->offs[d->E] = run;
  const int n = (int)d->experts.size();
  d->work_e.resize(n);
  d->work_slot.resize(n);
  d->work_wave.resize(n);
  d->misses.resize(n);
  int nm = 0, nw = 0;
  rc = cache_resolve(d->cache, step, layer, d->experts.data(), n, d->work_e.data(), d->work_slot.data(),
                     d->work_wave.data(), d->misses.data(), &nm, &nw);
  if (rc != MOE_OK) return dfail(rc, "moe_decoder_step: %s", moe_last_error());
  if (early_hits) {
    rc = update_slot_table(d, layer, n, nm, s);
    if (rc != MOE_OK) return rc;
    int hits = 0, rows = 0;
    for (int i = 0; i < n; ++i)
      if (d->work_slot[i] >= 0) {
        ++hits;
        rows += d->counts[d->work_e[i]];
      }
    // every expert of the step resident at its start: no fills and none run on the CPU (the resident list
    // then held all of them, so a fused launch has formed `out`)
    all_resident = nm == 0 && hits == n && n > 0;
    if (d->prof_every > 0 && all_resident && d->prof_calls++ % d->prof_every == 0 && prof_open) {
      const double a = d->dtype == MOE_DT_BF16 ? 2.0 : 4.0, h = d->wfmt == MOE_W_F32 ? 4.0 : 2.0;
      d->ev_bytes[d->ev_used] = (double)hits * (double)d->blob_bytes +
                                (double)rows * (d->H * a + 2.0 * d->I * h + d->H * 4.0) +
                                (fused ? (double)T * d->H * (out_dtype == MOE_DT_BF16 ? 2.0 : 4.0) : 0.0);
      ++d->ev_used;
    }
    // each wave's misses: their fills, then their FFN
    for (int w = 0; w < nw; ++w) {
      d->wave_misses.clear();
      for (int i = 0; i < nm; ++i)
        if (d->misses[i].wave == w) d->wave_misses.push_back(d->misses[i]);
      if (d->wave_misses.empty()) continue;
      hipEvent_t filled = nullptr;
      rc = cache_fill_enqueue(d->cache, d->wave_misses.data(), (int)d->wave_misses.size(), d->layer_pool.data(),
                              d->blob_stride, d->blob_bytes, d->slot_base, d->slot_stride, d->fill, stream, &filled,
                              w == 0 && !counts_event ? nullptr : (w == 0 ? d->ev_counts : nullptr),
                              w == 0 && !counts_event);
      if (rc != MOE_OK) {
        const std::string msg = moe_last_error();
        for (int i = 0; i < nm; ++i)
          if (d->misses[i].wave > w) (void)moe_cache_invalidate(d->cache, d->misses[i].key);
        return dfail(rc, "moe_decoder_step: %s", msg.c_str());
      }
      d->fills += (int64_t)d->wave_misses.size();
      if (filled) e = hipStreamWaitEvent(s, filled, 0);
      if (e != hipSuccess) {
        for (int i = 0; i < nm; ++i)
          if (d->misses[i].wave >= w) (void)moe_cache_invalidate(d->cache, d->misses[i].key);
        return dfail(MOE_EHIP, "moe_decoder_step: wait for fills: %s", hipGetErrorString(e));
      }
      d->work.clear();
      for (const moe_miss_t& m : d->wave_misses) {
        const int ex = m.key - layer * d->E;
        d->work.push_back(moe_work_t{ex, m.slot, d->offs[ex], d->counts[ex]});
      }
      rc = moe_ffn(x, d->dtype, b.perm_src, d->work.data(), (int)d->work.size(), d->slot_base, d->slot_stride,
                   d->wfmt, d->H, d->I, b.y_perm, b.ffn_ws, b.ffn_ws_bytes, MOE_FFN_AUTO, stream);
      if (rc != MOE_OK) return dfail(rc, "moe_decoder_step: %s", moe_last_error());
    }
  }
  if (!early_hits) d->slot_of_edits = ~0ull;  // this resolve's changes are not in the GPU copy
  for (int w = 0; w < nw && !early_hits; ++w) {
    d->wave_misses.clear();
    for (int i = 0; i < nm; ++i)
      if (d->misses[i].wave == w) d->wave_misses.push_back(d->misses[i]);
    hipEvent_t filled = nullptr;
    if (!d->wave_misses.empty()) {
      rc = cache_fill_enqueue(d->cache, d->wave_misses.data(), (int)d->wave_misses.size(), d->layer_pool.data(),
                              d->blob_stride, d->blob_bytes, d->slot_base, d->slot_stride, d->fill, stream, &filled,
                              nullptr, false);
      if (rc != MOE_OK) {
        // the fill call has unmapped this wave's misses that it could not copy; the later waves' misses
        // were never copied: unmap them too
        const std::string msg = moe_last_error();
        for (int i = 0; i < nm; ++i)
          if (d->misses[i].wave > w) (void)moe_cache_invalidate(d->cache, d->misses[i].key);
        return dfail(rc, "moe_decoder_step: %s", msg.c_str());
      }
      d->fills += (int64_t)d->wave_misses.size();
    }
    // the wave in access order: its hits, then its misses (the last wave_misses.size() items); the hits'
    // FFN runs while the misses are being copied, the misses' FFN once the copies are done
    int wave_items = 0;
    for (int i = 0; i < n; ++i) wave_items += d->work_wave[i] == w;
    const int n_miss_w = (int)d->wave_misses.size();
    const int split_at = filled ? wave_items - n_miss_w : wave_items;
    for (int part = 0; part < 2; ++part) {
      if (part == 1) {
        if (!filled) break;
        e = hipStreamWaitEvent(s, filled, 0);
        if (e != hipSuccess) {  // no reader would wait for this wave's copies, and later waves get none
          for (int i = 0; i < nm; ++i)
            if (d->misses[i].wave >= w) (void)moe_cache_invalidate(d->cache, d->misses[i].key);
          return dfail(MOE_EHIP, "moe_decoder_step: wait for fills: %s", hipGetErrorString(e));
        }
      }
      d->work.clear();
      int rows = 0, pos = 0;
      for (int i = 0; i < n; ++i) {
        if (d->work_wave[i] != w) continue;
        const bool take = part == 0 ? pos < split_at : pos >= split_at;
        ++pos;
        if (!take) continue;
        const int ex = d->work_e[i];
        d->work.push_back(moe_work_t{ex, d->work_slot[i], d->offs[ex], d->counts[ex]});
        rows += d->counts[ex];
      }
      if (d->work.empty()) continue;
      // profiled calls: the FFN of a whole layer-step whose experts were all resident
      const bool whole = nw == 1 && !filled;
      const bool prof = whole && d->prof_every > 0 && d->prof_calls++ % d->prof_every == 0;
      if (prof && record_ffn_event(d, true, s, 0) != MOE_OK)
        return dfail(MOE_EHIP, "moe_decoder_step: profiling event");
      rc = moe_ffn(x, d->dtype, b.perm_src, d->work.data(), (int)d->work.size(), d->slot_base, d->slot_stride,
                   d->wfmt, d->H, d->I, b.y_perm, b.ffn_ws, b.ffn_ws_bytes, MOE_FFN_AUTO, stream);
      if (rc != MOE_OK) return dfail(rc, "moe_decoder_step: %s", moe_last_error());
      if (prof) {
        const double a = d->dtype == MOE_DT_BF16 ? 2.0 : 4.0, h = d->wfmt == MOE_W_F32 ? 4.0 : 2.0;
        const double bytes = (double)d->work.size() * (double)d->blob_bytes +
                             (double)rows * (d->H * a + 2.0 * d->I * h + d->H * 4.0);
        if (record_ffn_event(d, false, s, bytes) != MOE_OK)
          return dfail(MOE_EHIP, "moe_decoder_step: profiling event");
      }
    }
  }
  // misses run on the CPU, straight from the pool, while the GPU works on the
  // rest; their rows of y_perm follow on the compute stream before the combine
  for (int i = 0; i < n; ++i) {
    if (d->work_slot[i] >= 0) continue;
    const int ex = d->work_e[i], rows = d->counts[ex], r0 = d->offs[ex];
    for (int r = 0; r < rows; ++r)
      std::memcpy(d->xg.data() + (size_t)r * d->H, d->x_host + (size_t)d->perm_host[r0 + r] * d->H,
                  sizeof(uint16_t) * d->H);
    const char* blob = static_cast<const char*>(d->layer_pool[layer]) + (size_t)ex * d->blob_stride;
    rc = moe_cpu_ffn(blob, d->wfmt, d->H, d->I, d->xg.data(), rows, d->y_host + (size_t)r0 * d->H, 0);
    if (rc != MOE_OK) return dfail(rc, "moe_decoder_step: %s", moe_last_error());
    e = hipMemcpyAsync(b.y_perm + (size_t)r0 * d->H, d->y_host + (size_t)r0 * d->H, sizeof(float) * rows * d->H,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return dfail(MOE_EHIP, "moe_decoder_step: CPU rows to the GPU: %s", hipGetErrorString(e));
    ++d->cpu_runs;
  }
  if (!(fused && all_resident)) {  // with every expert resident the fused launch has written `out`
    rc = moe_combine(b.y_perm, b.perm_pos, b.topk_w, T, d->k, d->H, out, out_dtype, stream);
    if (rc != MOE_OK) return dfail(rc, "moe_decoder_step: %s", moe_last_error());
  }
  if (n_miss) *n_miss = nm;
  return MOE_OK;
}

int moe_decoder_resize(moe_decoder_t* d, int S_new, void* slot_base, void* stream) {
  if (!d) return dfail(MOE_EINVAL, "moe_decoder_resize: null decoder");
  const int S_old = moe_cache_capacity(d->cache);
  int n_layers = 0;
  (void)moe_cache_layers(d->cache, &n_layers);
  // slots of the resident entries before the resize
  std::vector<std::pair<int, int>> resident;  // (key, slot)
  for (int key = 0; key < n_layers * d->E; ++key) {
    int sl = -1;
    if (moe_cache_slot_of(d->cache, key, &sl) == MOE_OK && sl >= 0) resident.emplace_back(key, sl);
  }
  std::vector<moe_move_t> moves(S_old > 0 ? S_old : 1);
  int nm = 0;
  int rc = moe_cache_resize(d->cache, S_new, moves.data(), (int)moves.size(), &nm);
  if (rc != MOE_OK) return dfail(rc, "moe_decoder_resize: %s", moe_last_error());
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* old_base = static_cast<char*>(d->slot_base);
  char* new_base = slot_base ? static_cast<char*>(slot_base) : old_base;
  hipError_t e = hipSuccess;
  for (int i = 0; i < nm && e == hipSuccess; ++i)
    e = hipMemcpyAsync(new_base + (size_t)moves[i].to_slot * d->slot_stride,
                       old_base + (size_t)moves[i].from_slot * d->slot_stride, d->blob_bytes,
                       hipMemcpyDeviceToDevice, s);
  if (new_base != old_base) {
    // entries that keep their slot still change buffer
    for (const auto& kv : resident) {
      int sl = -1;
      (void)moe_cache_slot_of(d->cache, kv.first, &sl);
      if (sl >= 0 && sl == kv.second && e == hipSuccess)
        e = hipMemcpyAsync(new_base + (size_t)sl * d->slot_stride, old_base + (size_t)sl * d->slot_stride,
                           d->blob_bytes, hipMemcpyDeviceToDevice, s);
    }
  }
  if (e != hipSuccess) return dfail(MOE_EHIP, "moe_decoder_resize: copy: %s", hipGetErrorString(e));
  d->slot_base = new_base;
  return MOE_OK;
}

int moe_decoder_profile(moe_decoder_t* d, int every) {
  if (!d || every < 0) return dfail(MOE_EINVAL, "moe_decoder_profile: null decoder or negative period");
  d->prof_every = every;
  d->prof_calls = 0;
  d->ev_used = 0;
  return MOE_OK;
}

int moe_decoder_ffn_stats(moe_decoder_t* d, double* bytes, double* ms, int64_t* launches) {
  if (!d || !bytes || !ms || !launches) return dfail(MOE_EINVAL, "moe_decoder_ffn_stats: null argument");
  double tb = 0, tm = 0;
  for (size_t i = 0; i < d->ev_used; ++i) {
    float m = 0;
    hipError_t e = hipEventSynchronize(d->ev_end[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&m, d->ev_begin[i], d->ev_end[i]);
    if (e != hipSuccess) return dfail(MOE_EHIP, "moe_decoder_ffn_stats: %s", hipGetErrorString(e));
    tb += d->ev_bytes[i];
    tm += m;
  }
  *bytes = tb;
  *ms = tm;
  *launches = (int64_t)d->ev_used;
  return MOE_OK;
}

int moe_decoder_fills(const moe_decoder_t* d, int64_t* fills) {
  if (!d || !fills) return dfail(MOE_EINVAL, "moe_decoder_fills: null argument");
  *fills = d->fills;
  return MOE_OK;
}

int moe_decoder_cpu_runs(const moe_decoder_t* d, int64_t* runs) {
  if (!d || !runs) return dfail(MOE_EINVAL, "moe_decoder_cpu_runs: null argument");
  *runs = d->cpu_runs;
  return MOE_OK;
}

}  // extern "C"
