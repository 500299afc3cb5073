// Host-only driver of the library's host code -- the shared LRU policy, the
// rule that a failed fill leaves its keys unmapped, and the CPU expert kernel
// -- built with g++ (no HIP) under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py, which compares
// what it prints with the oracle. Copies go through a mock copier that fails
// on request.
//
// Commands on stdin, one per line:
//   cache NKEYS S              a new policy of S slots over keys 0..NKEYS-1
//   split G C                  split the misses by the rates G (GPU) : C (CPU)
//   fail K                     the K-th copy from now fails (0: the next one)
//   step STEP LAYER E N e1..eN one layer-step: prints "rec step layer key hit
//                              slot victim wave" per access, then fills the
//                              GPU misses wave by wave as the decode driver
//                              does; a failed batch prints "drop key" for the
//                              keys it and the later waves leave unmapped
//   resize S                   prints "move key from to" per move
//   table                      prints "res key slot" per resident key
//   ffn BLOB X Y H I ROWS TH   moe_cpu_ffn on bf16 files (blob, x rows), y as fp32
#include <cstdarg>
#include <cstdio>
#include <fstream>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "../../routed_expert_layer_amd/csrc/lru_policy.hpp"

// The CPU kernel reports errors through the library's error setter, which
// lives in the HIP part of the library: this build supplies its own.
namespace moe {
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vfprintf(stderr, fmt, ap);
  va_end(ap);
  std::fputc('\n', stderr);
  return code;
}
}  // namespace moe

static std::vector<char> read_file(const std::string& path) {
  std::ifstream f(path, std::ios::binary);
  return std::vector<char>((std::istreambuf_iterator<char>(f)), std::istreambuf_iterator<char>());
}

int main() {
  moe::SharedLru* lru = nullptr;
  int n_keys = 0;
  long fail_at = -1;  // copies left before the failing one; -1: none fails
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "cache") {
      int S;
      in >> n_keys >> S;
      delete lru;
      lru = new moe::SharedLru(n_keys, S);
    } else if (cmd == "split") {
      long g, c;
      in >> g >> c;
      lru->set_split(g, c);
    } else if (cmd == "fail") {
      in >> fail_at;
    } else if (cmd == "step") {
      int step, layer, E, n;
      in >> step >> layer >> E >> n;
      std::vector<int32_t> keys(n);
      for (int i = 0; i < n; ++i) {
        int e;
        in >> e;
        keys[i] = layer * E + e;
      }
      std::vector<moe::Access> acc;
      lru->resolve(keys.data(), n, acc);
      int n_waves = 0;
      for (const moe::Access& a : acc) {
        std::printf("rec %d %d %d %d %d %d %d\n", step, layer, a.key, a.hit, a.slot, a.victim, a.wave);
        if (a.wave + 1 > n_waves) n_waves = a.wave + 1;
      }
      for (int w = 0; w < n_waves; ++w) {
        std::vector<int32_t> batch;
        for (const moe::Access& a : acc)
          if (!a.hit && a.slot >= 0 && a.wave == w) batch.push_back(a.key);
        const auto copy = [&](int) {
          if (fail_at < 0) return true;
          return fail_at-- != 0;
        };
        const int issued = moe::issue_fills(*lru, batch.data(), (int)batch.size(), copy);
        if (issued == (int)batch.size()) continue;
        for (size_t j = issued; j < batch.size(); ++j) std::printf("drop %d\n", batch[j]);
        for (const moe::Access& a : acc)  // later waves were never filled
          if (!a.hit && a.slot >= 0 && a.wave > w && lru->invalidate(a.key)) std::printf("drop %d\n", a.key);
        break;
      }
    } else if (cmd == "resize") {
      int S;
      in >> S;
      std::vector<moe::Move> mv;
      lru->resize(S, mv);
      for (const moe::Move& m : mv) std::printf("move %d %d %d\n", m.key, m.from, m.to);
    } else if (cmd == "table") {
      for (int k = 0; k < n_keys; ++k)
        if (lru->slot_of(k) >= 0) std::printf("res %d %d\n", k, lru->slot_of(k));
    } else if (cmd == "ffn") {
      std::string bp, xp, yp;
      int H, I, rows, th;
      in >> bp >> xp >> yp >> H >> I >> rows >> th;
      const std::vector<char> blob = read_file(bp), x = read_file(xp);
      std::vector<float> y((size_t)rows * H);
      const int rc = moe_cpu_ffn(blob.data(), MOE_W_BF16, H, I, x.data(), rows, y.data(), th);
      std::ofstream(yp, std::ios::binary).write(reinterpret_cast<const char*>(y.data()), y.size() * sizeof(float));
      std::printf("ffn %d\n", rc);
    } else {
      std::fprintf(stderr, "unknown command %s\n", cmd.c_str());
      return 2;
    }
    std::fflush(stdout);
  }
  delete lru;
  return 0;
}
