"""A textbook LRU cache on an ordered dict, used only to check the oracle's simulator.

It shares no code with oracle/lru.py: recency is the order of an OrderedDict
(move_to_end on a hit, popitem(last=False) for the victim), the way LRU is
usually written down.
"""
from collections import OrderedDict


class TextbookLRU:
    def __init__(self, S):
        self.S = S
        self.od = OrderedDict()          # key -> slot, least recent first
        self.free = list(range(S))

    def access(self, key):
        """Returns (hit, slot, victim)."""
        if key in self.od:
            self.od.move_to_end(key)
            return True, self.od[key], -1
        if self.free:
            slot = min(self.free)
            self.free.remove(slot)
            victim = -1
        else:
            victim, slot = self.od.popitem(last=False)
        self.od[key] = slot
        return False, slot, victim
