#include "lru_policy.hpp"

#include <algorithm>

namespace moe {

SharedLru::SharedLru(int n_keys, int S)
    : S_(S), key_slot_(n_keys, -1), slot_key_(S, -1), prev_(S, -1), next_(S, -1) {
  for (int s = 0; s < S; ++s) free_.insert(s);
}

void SharedLru::unlink(int s) {
  int p = prev_[s], n = next_[s];
  if (p >= 0) next_[p] = n; else lru_ = n;
  if (n >= 0) prev_[n] = p; else mru_ = p;
  prev_[s] = next_[s] = -1;
}

void SharedLru::push_mru(int s) {
  prev_[s] = mru_;
  next_[s] = -1;
  if (mru_ >= 0) next_[mru_] = s; else lru_ = s;
  mru_ = s;
}

void SharedLru::set_split(int64_t rate_gpu, int64_t rate_cpu) {
  rate_gpu_ = rate_gpu;
  rate_cpu_ = rate_cpu;
  missed_ = to_gpu_ = 0;
}

void SharedLru::resolve(const int32_t* keys, int n, std::vector<Access>& out) {
  // Hits are decided before any access of this layer-step is made.
  std::vector<int32_t> order;
  order.reserve(n);
  for (int i = 0; i < n; ++i) if (key_slot_[keys[i]] >= 0) order.push_back(keys[i]);
  const size_t n_hits = order.size();
  for (int i = 0; i < n; ++i) if (key_slot_[keys[i]] < 0) order.push_back(keys[i]);
  // GPU share of the misses, with the remainder carried across layer-steps
  missed_ += (int64_t)(order.size() - n_hits);
  const int64_t q = rate_gpu_ * missed_ / (rate_gpu_ + rate_cpu_) - to_gpu_;
  to_gpu_ += q;
  const size_t n_gpu = n_hits + (size_t)q;
  misses_ += (int64_t)(order.size() - n_gpu);  // CPU-run misses, recorded last
  for (size_t pos = 0; pos < n_gpu; ++pos) {
    const int32_t key = order[pos];
    Access a{key, pos < n_hits ? 1 : 0, -1, -1, static_cast<int32_t>(pos / S_)};
    if (a.hit) {
      a.slot = key_slot_[key];
      unlink(a.slot);
      ++hits_;
    } else {
      if (!free_.empty()) {
        a.slot = *free_.begin();
        free_.erase(free_.begin());
      } else {
        a.slot = lru_;
        unlink(a.slot);
        a.victim = slot_key_[a.slot];
        key_slot_[a.victim] = -1;
      }
      slot_key_[a.slot] = key;
      key_slot_[key] = a.slot;
      ++misses_;
    }
    push_mru(a.slot);
    out.push_back(a);
  }
  for (size_t pos = n_gpu; pos < order.size(); ++pos) out.push_back(Access{order[pos], 0, -1, -1, -1});
}

bool SharedLru::invalidate(int key) {
  int s = key_slot_[key];
  if (s < 0) return false;
  unlink(s);
  key_slot_[key] = -1;
  slot_key_[s] = -1;
  free_.insert(s);
  ++edits_;
  return true;
}

int issue_fills(SharedLru& lru, const int32_t* keys, int n, const std::function<bool(int)>& copy) {
  for (int i = 0; i < n; ++i) {
    if (copy(i)) continue;
    for (int j = i; j < n; ++j) (void)lru.invalidate(keys[j]);
    return i;
  }
  return n;
}

void plan_resize(const std::vector<int32_t>& slot_key, const std::vector<uint64_t>& recency, int S_new,
                 std::vector<int32_t>& new_key, std::vector<int32_t>& origin, std::vector<Move>& moves,
                 std::vector<int32_t>& evicted) {
  const int S_old = (int)slot_key.size();
  std::vector<int> occ;
  for (int s = 0; s < S_old; ++s)
    if (slot_key[s] >= 0) occ.push_back(s);
  std::sort(occ.begin(), occ.end(), [&](int a, int b) { return recency[a] > recency[b]; });
  std::vector<char> keep(S_old, 0);
  for (size_t i = 0; i < occ.size(); ++i) {
    if ((int)i < S_new) keep[occ[i]] = 1;
    else evicted.push_back(slot_key[occ[i]]);
  }
  new_key.assign(S_new, -1);
  origin.assign(S_new, -1);
  for (int s = 0; s < S_old && s < S_new; ++s)
    if (keep[s]) {
      new_key[s] = slot_key[s];
      origin[s] = s;
    }
  int next_free = 0;
  for (int s = S_new; s < S_old; ++s) {
    if (!keep[s]) continue;
    while (new_key[next_free] >= 0) ++next_free;  // a kept entry above S_new implies a free slot below
    new_key[next_free] = slot_key[s];
    origin[next_free] = s;
    moves.push_back(Move{slot_key[s], s, next_free});
  }
}

void SharedLru::resize(int S_new, std::vector<Move>& moves) {
  ++edits_;
  // recency rank of every occupied slot, from the list (least recent first)
  std::vector<uint64_t> rank(S_, 0);
  std::vector<int> order;  // occupied slots, least recent first
  uint64_t r = 1;
  for (int s = lru_; s >= 0; s = next_[s]) {
    rank[s] = r++;
    order.push_back(s);
  }
  std::vector<int32_t> new_key, origin, evicted;
  plan_resize(slot_key_, rank, S_new, new_key, origin, moves, evicted);
  for (int32_t k : evicted) key_slot_[k] = -1;
  std::vector<int> new_of(S_, -1);  // old slot -> new slot of kept entries
  for (int s = 0; s < S_new; ++s) {
    if (origin[s] >= 0) {
      new_of[origin[s]] = s;
      key_slot_[new_key[s]] = s;
    }
  }
  S_ = S_new;
  slot_key_ = new_key;
  prev_.assign(S_new, -1);
  next_.assign(S_new, -1);
  lru_ = mru_ = -1;
  for (int s : order)
    if (new_of[s] >= 0) push_mru(new_of[s]);
  free_.clear();
  for (int s = 0; s < S_new; ++s)
    if (slot_key_[s] < 0) free_.insert(s);
}

}  // namespace moe
