// Direct CPU execution of one routed expert from its blob in host memory (the
// pages' "CPU execution" of selected cache misses: page "FreeToken-rtx-4090",
// component table row "CPU" and section "Adaptive Misses"). The blob is read
// in the same fragment order the GPU uses, so the host pool needs no second
// layout.
//
// bf16 blob: P1 (2I rows x H) then P2 (H rows x I), 16-row tiles of 1 KiB
// fragments in K order; fragment byte 16 l .. 16 l + 15 holds row l % 16,
// K 32 c + 8 (l / 16) .. + 7. A 64-byte run of a fragment (lanes 4j .. 4j+3)
// is rows 4 (j % 4) .. + 3 at K group j / 4, eight values each: one
// vdpbf16ps against the eight activations of that K group, broadcast four
// times, leaves in lane i the partial sum of row 4 (j % 4) + i / 4 over the
// K pair i % 4. P1 rows interleave gate and up: row 4q + s of tile t is
// column 8t + 2q + s/2 of W1 (s even) or W3 (s odd).
#include <immintrin.h>

#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "moe_kernels.hpp"

namespace {

// Worker threads that spin briefly on a generation counter, then sleep.
class Pool {
 public:
  explicit Pool(int workers) {
    for (int i = 0; i < workers; ++i) th_.emplace_back([this, i] { loop(i + 1); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(m_);
      stop_ = true;
      gen_.fetch_add(1);
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  int workers() const { return (int)th_.size(); }
  // Runs f(index, count) on `count` participants (the caller is index 0).
  void run(int count, const std::function<void(int, int)>& f) {
    if (count > workers() + 1) count = workers() + 1;
    if (count <= 1) {
      f(0, 1);
      return;
    }
    job_ = &f;
    count_ = count;
    done_.store(0, std::memory_order_relaxed);
    {
      std::lock_guard<std::mutex> lk(m_);
      gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    f(0, count);
    while (done_.load(std::memory_order_acquire) < workers()) _mm_pause();
  }

 private:
  void loop(int id) {
    uint64_t seen = 0;
    for (;;) {
      int spins = 0;
      while (gen_.load(std::memory_order_acquire) == seen) {
        if (++spins < (1 << 16)) {
          _mm_pause();
        } else {
          std::unique_lock<std::mutex> lk(m_);
          cv_.wait(lk, [&] { return gen_.load(std::memory_order_acquire) != seen; });
        }
      }
      seen = gen_.load(std::memory_order_acquire);
      if (stop_) return;
      if (id < count_) (*job_)(id, count_);
      done_.fetch_add(1, std::memory_order_release);
    }
  }
  std::vector<std::thread> th_;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> done_{0};
  const std::function<void(int, int)>* job_ = nullptr;
  int count_ = 0;
  bool stop_ = false;
  std::mutex m_;
  std::condition_variable cv_;
};

Pool& pool() {
  static Pool p((int)std::thread::hardware_concurrency() > 1 ? (int)std::thread::hardware_concurrency() - 1 : 0);
  return p;
}

constexpr int kRB = 4;  // token rows per register block

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

inline float silu(float g) { return g / (1.0f + std::exp(-g)); }

// Sums of lanes 4i .. 4i+3 of v, i = 0..3.
inline void quad_sums(__m512 v, float out[4]) {
  alignas(64) float t[16];
  _mm512_store_ps(t, v);
  for (int i = 0; i < 4; ++i) out[i] = (t[4 * i] + t[4 * i + 1]) + (t[4 * i + 2] + t[4 * i + 3]);
}

// One 16-row tile: dot products of its rows (KC fragments at `frag`) with
// `nr` <= kRB activation rows act[r * ld .. + 32 KC] (bf16); res[r][16].
void tile_dot(const uint16_t* frag, int KC, const uint16_t* act, size_t ld, int nr, float res[kRB][16]) {
  __m512 acc[4][kRB];
  for (int q = 0; q < 4; ++q)
    for (int r = 0; r < kRB; ++r) acc[q][r] = _mm512_setzero_ps();
  for (int c = 0; c < KC; ++c) {
    const char* f = reinterpret_cast<const char*>(frag) + (size_t)c * 1024;
    for (int g = 0; g < 4; ++g) {
      __m512bh b[kRB];
      for (int r = 0; r < kRB; ++r) {
        const __m128i x8 = r < nr ? _mm_loadu_si128(reinterpret_cast<const __m128i*>(act + r * ld + 32 * c + 8 * g))
                                  : _mm_setzero_si128();
        b[r] = (__m512bh)_mm512_broadcast_i32x4(x8);
      }
      for (int q = 0; q < 4; ++q) {
        const __m512bh a = (__m512bh)_mm512_loadu_si512(f + 64 * q + 256 * g);
        for (int r = 0; r < kRB; ++r) acc[q][r] = _mm512_dpbf16_ps(acc[q][r], a, b[r]);
      }
    }
  }
  for (int r = 0; r < nr; ++r)
    for (int q = 0; q < 4; ++q) quad_sums(acc[q][r], &res[r][4 * q]);
}

}  // namespace

extern "C" {

int moe_cpu_ffn(const void* blob, int wfmt, int H, int I, const void* x, int rows, float* y, int threads) {
  if (!blob || (rows > 0 && (!x || !y)) || rows < 0) return moe::set_error(MOE_EINVAL, "moe_cpu_ffn: null pointer");
  if (wfmt != MOE_W_BF16 || H <= 0 || I <= 0 || H % 32 != 0 || I % 32 != 0)
    return moe::set_error(MOE_EINVAL, "moe_cpu_ffn: needs bf16 weights with H, I multiples of 32");
  if (rows == 0) return MOE_OK;
  if (threads <= 0) threads = pool().workers() + 1;
  const uint16_t* p1 = static_cast<const uint16_t*>(blob);
  const uint16_t* p2 = p1 + (size_t)2 * H * I;
  const uint16_t* xa = static_cast<const uint16_t*>(x);
  const int KC1 = H / 32, NT1 = 2 * I / 16, KC2 = I / 32, NT2 = H / 16;
  std::vector<uint16_t> h((size_t)rows * I);
  // gate/up and SwiGLU: h[r][i] = bf16(silu(x W1)[i] * (x W3)[i])
  pool().run(threads, [&](int id, int n) {
    float res[kRB][16];
    for (int t = (int)((long)NT1 * id / n); t < (int)((long)NT1 * (id + 1) / n); ++t)
      for (int r0 = 0; r0 < rows; r0 += kRB) {
        const int nr = rows - r0 < kRB ? rows - r0 : kRB;
        tile_dot(p1 + (size_t)t * KC1 * 512, KC1, xa + (size_t)r0 * H, (size_t)H, nr, res);
        for (int r = 0; r < nr; ++r)
          for (int q = 0; q < 4; ++q)
            for (int s2 = 0; s2 < 2; ++s2) {
              const float gv = res[r][4 * q + 2 * s2], uv = res[r][4 * q + 2 * s2 + 1];
              h[(size_t)(r0 + r) * I + 8 * t + 2 * q + s2] = f32_to_bf16_rne(silu(gv) * uv);
            }
      }
  });
  // down projection: y[r][n] = h[r] . W2[:, n]
  pool().run(threads, [&](int id, int n) {
    float res[kRB][16];
    for (int t = (int)((long)NT2 * id / n); t < (int)((long)NT2 * (id + 1) / n); ++t)
      for (int r0 = 0; r0 < rows; r0 += kRB) {
        const int nr = rows - r0 < kRB ? rows - r0 : kRB;
        tile_dot(p2 + (size_t)t * KC2 * 512, KC2, h.data() + (size_t)r0 * I, (size_t)I, nr, res);
        for (int r = 0; r < nr; ++r) std::memcpy(y + (size_t)(r0 + r) * H + 16 * t, res[r], 16 * sizeof(float));
      }
  });
  return MOE_OK;
}

int moe_cpu_threads(void) { return pool().workers() + 1; }

}  // extern "C"

namespace moe {

// Reads one byte of every 4 KiB page of [p, p + bytes) on all pool threads.
// Pinned memory that only the GPU has written pays a large cost on the CPU's
// first read of each page (measured: ~10x slower than later reads), which
// would otherwise land on the first CPU execution of every expert.
void cpu_touch_pages(const void* p, size_t bytes) {
  const volatile char* c = static_cast<const volatile char*>(p);
  const size_t pages = (bytes + 4095) / 4096;
  std::atomic<unsigned> sink{0};
  pool().run(pool().workers() + 1, [&](int id, int n) {
    unsigned acc = 0;
    for (size_t i = pages * id / n; i < pages * (id + 1) / n; ++i) acc += (unsigned char)c[i * 4096];
    sink.fetch_add(acc, std::memory_order_relaxed);
  });
}

}  // namespace moe
