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

// int4 and MXFP4 blobs: a 16-row tile is K/128 blocks of 1 KiB of 4-bit
// codes; block byte 16 l .. 16 l + 15 (lane l) holds four 32-bit words, word j
// being row l % 16 at K 128 g + 32 j + 8 (l / 16) .. + 7. A 64-byte run m of
// a block (lanes 4m .. 4m+3) is rows 4 (m % 4) .. + 3 at K group s = m / 4;
// its 16 words, turned into four vectors of bf16 pairs (pair p = the codes of
// K 2p and 2p + 1 of each word), meet the activation pairs of the same K in
// one vdpbf16ps each. Lane 4i + j of accumulator q then sums row 4q + i over
// its word j, so the per-block scales apply lane by lane and the four j lanes
// are added once at the end.
enum class Q4 { kInt4, kMxfp4 };

// Activation pairs for every (K block g, group s, pair p) of one row, as the
// 16 words the code vectors need (word 4i + j = the bf16 pair at K 128 g +
// 32 j + 8 s + 2 p), and, for int4, the row's sum over each K block.
struct Q4Act {
  std::vector<__m512i> pairs;  // [KG][4][4]
  std::vector<float> block_sum;  // [KG]
};

void q4_activations(const uint16_t* xr, int K, Q4Act& a) {
  const int KG = K / 128;
  a.pairs.resize((size_t)KG * 16);
  a.block_sum.resize(KG);
  for (int g = 0; g < KG; ++g) {
    float sum = 0.f;
    for (int k = 0; k < 128; ++k) {
      const uint32_t u = (uint32_t)xr[128 * g + k] << 16;
      float f;
      std::memcpy(&f, &u, 4);
      sum += f;
    }
    a.block_sum[g] = sum;
    for (int s = 0; s < 4; ++s)
      for (int p = 0; p < 4; ++p) {
        alignas(64) uint32_t w[16];
        for (int j = 0; j < 4; ++j) {
          uint32_t v;
          std::memcpy(&v, xr + 128 * g + 32 * j + 8 * s + 2 * p, 4);
          for (int i = 0; i < 4; ++i) w[4 * i + j] = v;
        }
        a.pairs[(size_t)(g * 4 + s) * 4 + p] = _mm512_load_si512(w);
      }
  }
}

// The four bf16-pair vectors of 16 code words. int4 (nibbles k0,k2,k4,k6,
// k1,k3,k5,k7, nibble n = q + 8): nibble n in the top mantissa bits of 1.0 is
// 1 + n/16 exactly, so a block's sum is 16 t - 24 u (u the activations' sum).
// MXFP4 (nibbles in K order): each nibble indexes the E2M1 values as bf16.
template <Q4 F>
inline void q4_codes_to_bf16(__m512i w, __m512i out[4]) {
  if constexpr (F == Q4::kInt4) {
    const __m512i m = _mm512_set1_epi32(0x00780078), one = _mm512_set1_epi32(0x3F803F80);
    out[0] = _mm512_ternarylogic_epi32(_mm512_slli_epi32(w, 3), m, one, 0xEA);  // (a & b) | c
    out[1] = _mm512_ternarylogic_epi32(_mm512_srli_epi32(w, 1), m, one, 0xEA);
    out[2] = _mm512_ternarylogic_epi32(_mm512_srli_epi32(w, 5), m, one, 0xEA);
    out[3] = _mm512_ternarylogic_epi32(_mm512_srli_epi32(w, 9), m, one, 0xEA);
  } else {
    // E2M1 codes 0..15 as bf16: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives
    const __m512i lut = _mm512_set_epi16(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, (short)0xC0C0, (short)0xC080,
                                         (short)0xC040, (short)0xC000, (short)0xBFC0, (short)0xBF80, (short)0xBF00,
                                         (short)0x8000, 0x40C0, 0x4080, 0x4040, 0x4000, 0x3FC0, 0x3F80, 0x3F00, 0);
    const __m512i lo = _mm512_set1_epi32(0xF), hi = _mm512_set1_epi32(0xF0000);
    for (int p = 0; p < 4; ++p) {
      const __m512i t = _mm512_srli_epi32(w, 8 * p);
      const __m512i idx = _mm512_ternarylogic_epi32(_mm512_and_si512(t, lo), _mm512_slli_epi32(t, 12), hi, 0xF8);
      out[p] = _mm512_permutexvar_epi16(idx, lut);  // a | (b & c)
    }
  }
}

// One 16-row tile of an int4 or MXFP4 matrix (KG blocks at `codes`, their
// scale blocks at `scales`) against nr <= kRB rows of activations; res[r][16].
template <Q4 F>
void tile_dot_q4(const char* codes, const char* scales, int KG, const Q4Act* act, int nr, float res[kRB][16]) {
  __m512 tot[4][kRB];
  for (int q = 0; q < 4; ++q)
    for (int r = 0; r < kRB; ++r) tot[q][r] = _mm512_setzero_ps();
  // lane 4i + j of scale vector q belongs to row 4q + i
  alignas(64) int32_t rowidx[4][16];
  for (int q = 0; q < 4; ++q)
    for (int l = 0; l < 16; ++l) rowidx[q][l] = 4 * q + l / 4;
  for (int g = 0; g < KG; ++g) {
    __m512 acc[4][kRB];
    for (int q = 0; q < 4; ++q)
      for (int r = 0; r < kRB; ++r) acc[q][r] = _mm512_setzero_ps();
    const char* blk = codes + (size_t)g * 1024;
    for (int m = 0; m < 16; ++m) {
      __m512i a[4];
      q4_codes_to_bf16<F>(_mm512_loadu_si512(blk + 64 * m), a);
      const int q = m & 3, s = m >> 2;
      for (int r = 0; r < nr; ++r) {
        const __m512i* b = &act[r].pairs[(size_t)(g * 4 + s) * 4];
        for (int p = 0; p < 4; ++p) acc[q][r] = _mm512_dpbf16_ps(acc[q][r], (__m512bh)a[p], (__m512bh)b[p]);
      }
    }
    if constexpr (F == Q4::kInt4) {
      // 16 fp16 scales, row r in lane r
      const __m512 sc = _mm512_cvtph_ps(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(scales + 32 * g)));
      for (int q = 0; q < 4; ++q) {
        const __m512 sq = _mm512_permutexvar_ps(_mm512_load_si512(rowidx[q]), sc);
        for (int r = 0; r < nr; ++r) {
          // the four j lanes of a row share -24 u
          const __m512 t = _mm512_fmadd_ps(acc[q][r], _mm512_set1_ps(16.f), _mm512_set1_ps(-6.f * act[r].block_sum[g]));
          tot[q][r] = _mm512_fmadd_ps(sq, t, tot[q][r]);
        }
      }
    } else {
      // byte 4 r + j of the 64-byte block: row r, K chunk j; byte 16 q + l is lane l of vector q
      for (int q = 0; q < 4; ++q) {
        const __m512i e = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(scales + 64 * g + 16 * q)));
        const __m512 sq = _mm512_castsi512_ps(_mm512_slli_epi32(e, 23));  // 2^(e - 127)
        for (int r = 0; r < nr; ++r) tot[q][r] = _mm512_fmadd_ps(sq, acc[q][r], tot[q][r]);
      }
    }
  }
  for (int r = 0; r < nr; ++r)
    for (int q = 0; q < 4; ++q) quad_sums(tot[q][r], &res[r][4 * q]);
}

template <Q4 F>
void cpu_ffn_q4(const char* blob, int wfmt, int H, int I, const uint16_t* xa, int rows, float* y, int threads) {
  const moe::BlobLayout lay = moe::blob_layout(wfmt, H, I);
  const size_t sblk = F == Q4::kInt4 ? 32 : 64;  // scale bytes per tile and K block
  const int KG1 = H / 128, NT1 = 2 * I / 16, KG2 = I / 128, NT2 = H / 16;
  std::vector<Q4Act> ax(rows), ah(rows);
  for (int r = 0; r < rows; ++r) q4_activations(xa + (size_t)r * H, H, ax[r]);
  std::vector<uint16_t> h((size_t)rows * I);
  pool().run(threads, [&](int id, int n) {
    float res[kRB][16];
    for (int t = (int)((long)NT1 * id / n); t < (int)((long)NT1 * (id + 1) / n); ++t)
      for (int r0 = 0; r0 < rows; r0 += kRB) {
        const int nr = rows - r0 < kRB ? rows - r0 : kRB;
        tile_dot_q4<F>(blob + lay.p1 + (size_t)t * KG1 * 1024, blob + lay.p1s + (size_t)t * KG1 * sblk, KG1,
                       ax.data() + r0, nr, res);
        for (int r = 0; r < nr; ++r)
          for (int q = 0; q < 4; ++q)
            for (int s2 = 0; s2 < 2; ++s2) {
              const float gv = res[r][4 * q + 2 * s2], uv = res[r][4 * q + 2 * s2 + 1];
              h[(size_t)(r0 + r) * I + 8 * t + 2 * q + s2] = f32_to_bf16_rne(silu(gv) * uv);
            }
      }
  });
  for (int r = 0; r < rows; ++r) q4_activations(h.data() + (size_t)r * I, I, ah[r]);
  pool().run(threads, [&](int id, int n) {
    float res[kRB][16];
    for (int t = (int)((long)NT2 * id / n); t < (int)((long)NT2 * (id + 1) / n); ++t)
      for (int r0 = 0; r0 < rows; r0 += kRB) {
        const int nr = rows - r0 < kRB ? rows - r0 : kRB;
        tile_dot_q4<F>(blob + lay.p2 + (size_t)t * KG2 * 1024, blob + lay.p2s + (size_t)t * KG2 * sblk, KG2,
                       ah.data() + r0, nr, res);
        for (int r = 0; r < nr; ++r) std::memcpy(y + (size_t)(r0 + r) * H + 16 * t, res[r], 16 * sizeof(float));
      }
  });
}

}  // namespace

extern "C" {

int moe_cpu_ffn(const void* blob, int wfmt, int H, int I, const void* x, int rows, float* y, int threads) {
  if (!blob || (rows > 0 && (!x || !y)) || rows < 0) return moe::set_error(MOE_EINVAL, "moe_cpu_ffn: null pointer");
  const bool q4 = wfmt == MOE_W_INT4 || wfmt == MOE_W_MXFP4;
  if ((wfmt != MOE_W_BF16 && !q4) || H <= 0 || I <= 0 || H % (q4 ? 128 : 32) != 0 || I % (q4 ? 128 : 32) != 0)
    return moe::set_error(MOE_EINVAL,
                          "moe_cpu_ffn: needs bf16 weights with H, I multiples of 32, or int4 / MXFP4 weights "
                          "with H, I multiples of 128");
  if (rows == 0) return MOE_OK;
  if (threads <= 0) threads = pool().workers() + 1;
  if (q4) {
    const char* b = static_cast<const char*>(blob);
    const uint16_t* xq = static_cast<const uint16_t*>(x);
    if (wfmt == MOE_W_INT4)
      cpu_ffn_q4<Q4::kInt4>(b, wfmt, H, I, xq, rows, y, threads);
    else
      cpu_ffn_q4<Q4::kMxfp4>(b, wfmt, H, I, xq, rows, y, threads);
    return MOE_OK;
  }
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
