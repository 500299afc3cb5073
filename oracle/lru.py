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
    def __init__(self, S):
        assert S >= 1
        self.S = S
        self.slot_key = [-1] * S
        self.last_use = [0] * S
        self.key_slot = {}
        self.clock = 0
        self.trace = []

    def resolve(self, step, layer, E, experts):
        """Run one layer-step. Returns (waves, records).

        waves: list of lists of (expert, slot) in access order.
        records: one TraceRec per accessed key (also appended to self.trace).
        """
        keys = sorted({layer * E + int(e) for e in experts})
        hit_set = {kk for kk in keys if kk in self.key_slot}
        seq = [kk for kk in keys if kk in hit_set] + [kk for kk in keys if kk not in hit_set]
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
        self.trace.extend(recs)
        return waves, recs
