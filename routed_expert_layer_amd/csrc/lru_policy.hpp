// Shared LRU policy over (layer, expert) keys: host-only C++, no HIP.
//
// Page "FreeToken-rtx-4090", section "How the MoE Memory Hierarchy Works": a
// cache entry is a logical layer-and-expert pair and decode keeps recently
// selected experts in one LRU cache shared across layers and tokens. One
// layer-step touches its working set hits-first then misses, each ascending;
// a miss takes the lowest free slot, else the least recently used entry's
// slot; accesses are cut into waves of at most S entries. Misses may be split
// between GPU fills and CPU execution (section "Adaptive Misses"): of all
// misses so far, floor(g * count / (g + c)) go to the GPU, the lowest keys of
// each layer-step first; CPU-run misses are not cached.
#pragma once
#include <cstdint>
#include <functional>
#include <set>
#include <vector>

namespace moe {

struct Access {
  int32_t key, hit, slot, victim, wave;
};

struct Move {
  int32_t key, from, to;
};

// Resize of a slot table at a safe point (page "FreeToken-benchmark", section
// "Elastic Cache"): the min(S_new, resident) most recent entries are kept
// (recency[s]: larger = more recent, for occupied slots); a kept entry below
// S_new stays in its slot, the kept entries at or above S_new move, in
// ascending old slot, to the lowest free slots below S_new. Outputs:
// new_key[S_new] (-1 free), origin[S_new] (old slot of each new slot's entry,
// -1 if free), the moves, and the keys evicted.
void plan_resize(const std::vector<int32_t>& slot_key, const std::vector<uint64_t>& recency, int S_new,
                 std::vector<int32_t>& new_key, std::vector<int32_t>& origin, std::vector<Move>& moves,
                 std::vector<int32_t>& evicted);

class SharedLru {
 public:
  SharedLru(int n_keys, int S);
  // One layer-step over ascending unique keys; appends to `out` the GPU
  // accesses in access order, then the CPU-run misses (slot, victim, wave -1).
  void resolve(const int32_t* keys, int n, std::vector<Access>& out);
  // Rates (any common unit) of GPU fills and CPU execution; resets the count.
  void set_split(int64_t rate_gpu, int64_t rate_cpu);
  bool splits() const { return rate_cpu_ > 0; }
  int slot_of(int key) const { return key_slot_[key]; }
  bool invalidate(int key);  // returns false if the key is not resident
  // Resize to S_new slots (plan_resize); recency order kept. Appends the moves.
  void resize(int S_new, std::vector<Move>& moves);
  int capacity() const { return S_; }
  // Number of changes to the slot table made other than by resolve
  // (invalidations and resizes): a copy of the table kept elsewhere is stale
  // once this moves.
  uint64_t edits() const { return edits_; }
  int64_t hits() const { return hits_; }
  int64_t misses() const { return misses_; }

 private:
  void unlink(int slot);
  void push_mru(int slot);
  int S_;
  std::vector<int32_t> key_slot_;  // key -> slot or -1
  std::vector<int32_t> slot_key_;  // slot -> key or -1
  std::vector<int32_t> prev_, next_;  // recency list over occupied slots
  int lru_ = -1, mru_ = -1;
  std::set<int> free_;
  int64_t hits_ = 0, misses_ = 0;
  int64_t rate_gpu_ = 1, rate_cpu_ = 0, missed_ = 0, to_gpu_ = 0;
  uint64_t edits_ = 0;
};

// Issues the copies of one batch of misses, in order, through copy(i) (false:
// the copy of miss i could not be issued). An entry is never left resident
// without its blob (page "FreeToken-rtx-4090", component table, row "PCIe
// link": a miss moves as one complete expert): at the first failure, that
// miss's key and the keys of every later miss of the batch are dropped from
// the cache (their slots become free); the misses issued before it stay
// resident. Returns the number of copies issued.
int issue_fills(SharedLru& lru, const int32_t* keys, int n, const std::function<bool(int)>& copy);

}  // namespace moe
