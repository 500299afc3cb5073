"""Shared LRU expert-cache simulator -- TEST INFRASTRUCTURE ONLY.

Follows page "FreeToken-rtx-4090": a cache entry is one logical
(layer, expert) pair (section "How the MoE Memory Hierarchy Works"), and decode
keeps recently selected experts in a single LRU cache shared across layers
and tokens that follows the current routing (same section, the decode
paragraph, and page "FreeToken-benchmark", section "How FreeToken Serves Large
MoE Models"). The pages do not say in which order one layer-step's experts
touch the cache, so this simulator takes the following reading:

  * key = layer * E + expert; the working set W of a layer-step is the
    ascending list of keys of experts with at least one routed token;
  * hits H = W keys resident when the layer-step starts, misses M = the rest;
    the access order is H ascending, then M ascending, and each access is
    ordinary least-recently-used bookkeeping;
  * a miss takes the lowest-numbered free slot, else the slot of the least
    recently used entry (its victim);
  * the accesses are cut into waves of at most S consecutive entries; the
    experts of one wave are all resident together, and a wave is executed
    before the next wave's misses are filled;
  * the cache starts empty.

Misses may also be executed on the CPU straight from the host pool instead of
being filled (page "FreeToken-rtx-4090", component table rows "CPU" and "PCIe
link", section "Adaptive Misses"; page "FreeToken-benchmark", "Adaptive
Misses"): the runtime measures the PCIe fill rate and the host's expert
processing rate and sends the share rate_gpu / (rate_gpu + rate_cpu) of the
misses to the GPU. The pages give neither the rounding nor which misses go
where; reading taken here:

  * the share is realised with a carried remainder: the number of misses sent
    to the GPU up to and including a layer-step is floor(rate_gpu * (misses up
    to it) / (rate_gpu + rate_cpu)), so single-miss layer-steps do not all
    round the same way;
  * of one layer-step's misses (ascending), the lowest q go to the GPU; the
    others run on the CPU, are not cached and do not touch the recency order;
  * the GPU accesses (hits, then GPU misses) form the waves as above; CPU
    misses are recorded after them with slot, victim and wave -1.

rate_cpu = 0 (the default) fills every miss.

The cache can be resized at a safe point, between layer-steps (page
"FreeToken-rtx-4090", runtime layer table, row "GPU memory": cache capacity can
change during runtime, and the phase table, row "Long sessions"; page
"FreeToken-benchmark", section "Elastic Cache": capacity is rebuilt without
reloading the host pool). The pages give no procedure; reading taken here:

  * resizing to S' slots keeps the min(S', resident) most recently used
    entries, with their recency order, and evicts the others (no trace
    records; the pool is untouched);
  * a kept entry in a slot below S' stays in its slot; the kept entries in
    slots at or above S' move, in ascending order of their old slot, to the
    lowest free slots below S' (each move is one copy of a blob);
  * growing adds free slots and moves nothing.

It keeps explicit per-slot last-use stamps rather than an ordered container,
so that the tests can check it against a textbook ordered-dict LRU.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class TraceRec:
    step: int
    layer: int
    key: int
    hit: int
    slot: int
    victim: int
    wave: int


class SharedLRU:
    def __init__(self, S, rate_gpu=1, rate_cpu=0):
        assert S >= 1
        self.S = S
        self.slot_key = [-1] * S
        self.last_use = [0] * S
        self.key_slot = {}
        self.clock = 0
        self.trace = []
        self.set_split(rate_gpu, rate_cpu)

    def set_split(self, rate_gpu, rate_cpu):
        """Integer rates; the share of misses filled is rate_gpu / (rate_gpu + rate_cpu)."""
        assert rate_gpu >= 0 and rate_cpu >= 0 and rate_gpu + rate_cpu > 0
        self.rate_gpu, self.rate_cpu = int(rate_gpu), int(rate_cpu)
        self.missed = 0   # misses seen since the split was set
        self.to_gpu = 0   # of which sent to the GPU

    def resolve(self, step, layer, E, experts):
        """Run one layer-step. Returns (waves, records).

        waves: list of lists of (expert, slot) in access order (GPU work).
        records: one TraceRec per key of the working set (also appended to
        self.trace); misses run on the CPU have slot -1.
        """
        keys = sorted({layer * E + int(e) for e in experts})
        hit_set = {kk for kk in keys if kk in self.key_slot}
        missing = [kk for kk in keys if kk not in hit_set]
        self.missed += len(missing)
        q = self.rate_gpu * self.missed // (self.rate_gpu + self.rate_cpu) - self.to_gpu
        self.to_gpu += q
        seq = [kk for kk in keys if kk in hit_set] + missing[:q]
        waves, recs = [], []
        for pos, key in enumerate(seq):
            wave = pos // self.S
            if wave == len(waves):
                waves.append([])
            self.clock += 1
            if key in hit_set:
                slot, victim = self.key_slot[key], -1
            else:
                free = [s for s in range(self.S) if self.slot_key[s] == -1]
                if free:
                    slot, victim = free[0], -1
                else:
                    slot = min(range(self.S), key=lambda s: self.last_use[s])
                    victim = self.slot_key[slot]
                    del self.key_slot[victim]
                self.slot_key[slot] = key
                self.key_slot[key] = slot
            self.last_use[slot] = self.clock
            waves[wave].append((key - layer * E, slot))
            recs.append(TraceRec(step, layer, key, int(key in hit_set), slot, victim, wave))
        for key in missing[q:]:  # executed on the CPU: not cached
            recs.append(TraceRec(step, layer, key, 0, -1, -1, -1))
        self.trace.extend(recs)
        return waves, recs

    def drop(self, key):
        """Unmap a key whose fill failed: its slot becomes free, so the next miss
        takes it if it is the lowest free slot. Page "FreeToken-rtx-4090",
        component table, row "PCIe link": a miss moves as one complete expert,
        so an entry whose copy did not happen must not stay resident. Returns
        False if the key was not resident."""
        slot = self.key_slot.pop(key, None)
        if slot is None:
            return False
        self.slot_key[slot] = -1
        self.last_use[slot] = 0
        return True

    def resize(self, S_new):
        """Resize to S_new slots at a safe point. Returns the moves [(key, old slot, new slot)]."""
        assert S_new >= 1
        occupied = [sl for sl in range(self.S) if self.slot_key[sl] != -1]
        keep = set(sorted(occupied, key=lambda sl: self.last_use[sl], reverse=True)[:S_new])
        for sl in occupied:
            if sl not in keep:
                del self.key_slot[self.slot_key[sl]]
                self.slot_key[sl] = -1
                self.last_use[sl] = 0
        new_key, new_use = [-1] * S_new, [0] * S_new
        for sl in range(min(self.S, S_new)):
            new_key[sl], new_use[sl] = self.slot_key[sl], self.last_use[sl]
        free = [sl for sl in range(S_new) if new_key[sl] == -1]
        moves = []
        for sl in range(S_new, self.S):
            if self.slot_key[sl] != -1:
                d = free.pop(0)
                new_key[d], new_use[d] = self.slot_key[sl], self.last_use[sl]
                self.key_slot[new_key[d]] = d
                moves.append((new_key[d], sl, d))
        self.S, self.slot_key, self.last_use = S_new, new_key, new_use
        return moves
