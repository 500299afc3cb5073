"""Pins for the oracle's shared LRU cache simulator.

Checked against a textbook ordered-dict LRU (tests/textbook_lru.py) fed the
same access order, and against cases whose hit counts are known in closed form.
"""
import numpy as np
import pytest

import oracle
from tests.textbook_lru import TextbookLRU


def _drive_both(S, E, L, steps, seed, max_active):
    r = np.random.default_rng(seed)
    sim = oracle.SharedLRU(S)
    tb = TextbookLRU(S)
    for step in range(steps):
        for layer in range(L):
            n = int(r.integers(1, max_active + 1))
            experts = sorted(r.choice(E, size=n, replace=False).tolist())
            waves, recs = sim.resolve(step, layer, E, experts)
            keys = [layer * E + e for e in experts]
            hits0 = [kk for kk in keys if kk in tb.od]
            seq = sorted(hits0) + sorted(kk for kk in keys if kk not in tb.od)
            assert [rc.key for rc in recs] == seq
            for pos, (rc, kk) in enumerate(zip(recs, seq)):
                hit, slot, victim = tb.access(kk)
                assert (rc.hit, rc.slot, rc.victim, rc.wave) == (int(hit), slot, victim, pos // S)
            # each wave's experts are resident together when that wave runs
            for w in waves:
                assert len(w) <= S
                assert len({s for _, s in w}) == len(w)
    return sim


@pytest.mark.parametrize("S,E,L,max_active", [(8, 16, 1, 14), (4, 10, 3, 6), (16, 32, 4, 10), (1, 5, 2, 3)])
def test_lru_matches_textbook(S, E, L, max_active):
    _drive_both(S, E, L, steps=60, seed=S * 100 + E, max_active=max_active)


def test_lru_cyclic_s_plus_one_never_hits():
    S = 5
    sim = oracle.SharedLRU(S)
    for step in range(40):
        _, recs = sim.resolve(step, 0, 100, [step % (S + 1)])
        assert recs[0].hit == 0
        if step >= S:
            assert recs[0].victim == (step + 1) % (S + 1)  # the least recent key is the next one wanted


def test_lru_compulsory_only():
    S, E = 16, 12
    sim = oracle.SharedLRU(S)
    r = np.random.default_rng(3)
    for step in range(50):
        sim.resolve(step, 0, E, sorted(r.choice(E, 4, replace=False).tolist()))
    misses = sum(1 for rc in sim.trace if not rc.hit)
    assert misses == len({rc.key for rc in sim.trace})  # <= S distinct keys: only first-touch misses


def test_lru_working_set_resident_after_step():
    S, E, L = 8, 32, 3
    sim = oracle.SharedLRU(S)
    r = np.random.default_rng(4)
    for step in range(30):
        for layer in range(L):
            ex = sorted(r.choice(E, int(r.integers(1, S + 1)), replace=False).tolist())
            sim.resolve(step, layer, E, ex)
            assert all(layer * E + e in sim.key_slot for e in ex)


def test_lru_waves_and_hits_first():
    S, E = 3, 10
    sim = oracle.SharedLRU(S)
    sim.resolve(0, 0, E, [1, 2])
    waves, recs = sim.resolve(1, 0, E, [0, 1, 2, 3, 4, 5])
    # hits (1, 2) first, then misses ascending; waves of S consecutive accesses
    assert [rc.key for rc in recs] == [1, 2, 0, 3, 4, 5]
    assert [rc.wave for rc in recs] == [0, 0, 0, 1, 1, 1]
    assert [rc.hit for rc in recs] == [1, 1, 0, 0, 0, 0]
    # wave 1 evicts the entries of wave 0, least recent first
    assert [rc.victim for rc in recs[3:]] == [1, 2, 0]
    assert waves == [[(1, 0), (2, 1), (0, 2)], [(3, 0), (4, 1), (5, 2)]]


# ---------------------------------------------------------------------------
# Misses split between GPU fills and CPU execution


@pytest.mark.parametrize("S,E,L,max_active,g,c", [(8, 16, 1, 14, 1, 3), (4, 10, 3, 6, 56, 165), (16, 32, 4, 10, 2, 1),
                                                  (1, 5, 2, 3, 5, 7), (8, 16, 2, 6, 1, 0)])
def test_split_against_textbook_and_closed_form(S, E, L, max_active, g, c):
    """GPU-bound accesses follow a textbook LRU that never sees the CPU-run keys;
    the filled share is floor(g * misses / (g + c)) after every layer-step."""
    r = np.random.default_rng(S * 7 + E + g)
    sim = oracle.SharedLRU(S, g, c)
    tb = TextbookLRU(S)
    from fractions import Fraction
    credit = Fraction(0)  # carried remainder, an independent statement of the rounding
    missed = filled = 0
    for step in range(60):
        for layer in range(L):
            n = int(r.integers(1, max_active + 1))
            experts = sorted(r.choice(E, size=n, replace=False).tolist())
            waves, recs = sim.resolve(step, layer, E, experts)
            keys = [layer * E + e for e in experts]
            hits0 = sorted(kk for kk in keys if kk in tb.od)
            miss0 = sorted(kk for kk in keys if kk not in tb.od)
            missed += len(miss0)
            credit += len(miss0) * Fraction(g, g + c)
            q = int(credit)  # floor (credit >= 0)
            credit -= q
            filled += q
            gpu, cpu = hits0 + miss0[:q], miss0[q:]
            assert [rc.key for rc in recs] == gpu + cpu
            for pos, (rc, kk) in enumerate(zip(recs, gpu)):
                hit, slot, victim = tb.access(kk)
                assert (rc.hit, rc.slot, rc.victim, rc.wave) == (int(hit), slot, victim, pos // S)
            for rc in recs[len(gpu):]:
                assert (rc.hit, rc.slot, rc.victim, rc.wave) == (0, -1, -1, -1)
                assert rc.key not in tb.od  # never cached
            assert sum(len(w) for w in waves) == len(gpu)
    assert filled == g * missed // (g + c)


def test_split_all_cpu_never_fills():
    sim = oracle.SharedLRU(4, 0, 1)
    for step in range(10):
        _, recs = sim.resolve(step, 0, 8, [1, 3, 5])
        assert all(rc.slot == -1 and rc.hit == 0 for rc in recs)
    assert sim.key_slot == {}


def test_split_cpu_misses_leave_cache_untouched():
    """Replaying only the GPU-bound experts through an unsplit simulator gives the same GPU records."""
    r = np.random.default_rng(5)
    sim = oracle.SharedLRU(6, 1, 2)
    plain = oracle.SharedLRU(6)
    for step in range(80):
        experts = sorted(r.choice(20, size=int(r.integers(1, 9)), replace=False).tolist())
        _, recs = sim.resolve(step, 0, 20, experts)
        gpu = [rc for rc in recs if rc.slot >= 0]
        _, recs2 = plain.resolve(step, 0, 20, sorted(rc.key for rc in gpu))
        assert [(rc.key, rc.hit, rc.slot, rc.victim, rc.wave) for rc in gpu] == \
            [(rc.key, rc.hit, rc.slot, rc.victim, rc.wave) for rc in recs2]


def _textbook_after(sim, tb, S_new):
    """A textbook LRU of S_new slots holding the oracle's kept entries, in the textbook's recency order."""
    t2 = TextbookLRU(S_new)
    order = list(tb.od.keys())[-S_new:] if S_new < len(tb.od) else list(tb.od.keys())
    for k in order:
        t2.od[k] = sim.key_slot[k]
    t2.free = [s for s in range(S_new) if s not in set(t2.od.values())]
    return t2


@pytest.mark.parametrize("S,S_new,E,L", [(16, 5, 32, 2), (8, 3, 12, 1), (6, 6, 10, 2), (4, 9, 12, 2), (8, 1, 9, 1)])
def test_resize_keeps_most_recent_and_continues_as_textbook_lru(S, S_new, E, L):
    r = np.random.default_rng(S * 31 + S_new)
    sim = oracle.SharedLRU(S)
    tb = TextbookLRU(S)

    def run(steps, step0, cap):
        for step in range(step0, step0 + steps):
            for layer in range(L):
                n = int(r.integers(1, min(cap, E) + 1))
                experts = sorted(r.choice(E, size=n, replace=False).tolist())
                _, recs = sim.resolve(step, layer, E, experts)
                for rc in recs:
                    hit, slot, victim = tb.access(rc.key)
                    assert (rc.hit, rc.slot, rc.victim) == (int(hit), slot, victim)

    run(20, 0, S)
    before = dict(sim.key_slot)
    recent = list(tb.od.keys())[-S_new:] if S_new < len(tb.od) else list(tb.od.keys())
    moves = sim.resize(S_new)
    # the survivors are exactly the S_new most recently used keys
    assert set(sim.key_slot) == set(recent)
    # moves take entries from slots >= S_new to distinct free slots < S_new; the others stay put
    targets = [d for _, _, d in moves]
    assert all(f >= S_new and d < S_new and before[k] == f for k, f, d in moves)
    assert len(set(targets)) == len(targets)
    stay = {k: s for k, s in before.items() if k in sim.key_slot and s < S_new}
    assert all(sim.key_slot[k] == s for k, s in stay.items())
    assert not set(targets) & set(stay.values())
    if S_new >= S:
        assert moves == []
    # afterwards the cache behaves as a textbook LRU of S_new slots holding those keys
    tb = _textbook_after(sim, tb, S_new)
    run(20, 20, S_new)


@pytest.mark.parametrize("S,E,L,max_active,seed", [(8, 16, 1, 14, 1), (6, 24, 2, 6, 2), (3, 9, 3, 4, 3)])
def test_drop_matches_textbook_with_key_deleted(S, E, L, max_active, seed):
    """A dropped key (failed fill) leaves the cache as a textbook LRU from which
    that key was deleted: same hits, slots and victims afterwards."""
    r = np.random.default_rng(seed)
    sim = oracle.SharedLRU(S)
    tb = TextbookLRU(S)
    dropped = 0
    for step in range(40):
        for layer in range(L):
            n = int(r.integers(1, max_active + 1))
            experts = sorted(r.choice(E, size=n, replace=False).tolist())
            _, recs = sim.resolve(step, layer, E, experts)
            for rc in recs:
                hit, slot, victim = tb.access(rc.key)
                assert (rc.hit, rc.slot, rc.victim) == (int(hit), slot, victim)
            # drop the misses of this layer-step from a random position on, as a failed batch of fills does
            misses = [rc.key for rc in recs if not rc.hit]
            if misses and r.random() < 0.3:
                for key in misses[int(r.integers(0, len(misses))):]:
                    slot = tb.od.pop(key)
                    tb.free.append(slot)
                    assert sim.drop(key)
                    assert key not in sim.key_slot and sim.slot_key[slot] == -1
                    dropped += 1
    assert dropped > 0
    assert not sim.drop(E * L)  # never resident


def test_drop_frees_lowest_slot_for_next_miss():
    sim = oracle.SharedLRU(4)
    sim.resolve(0, 0, 8, [0, 1, 2, 3])          # slots 0..3
    assert sim.drop(1)                           # slot 1 free
    _, recs = sim.resolve(1, 0, 8, [5])
    assert (recs[0].hit, recs[0].slot, recs[0].victim) == (0, 1, -1)
    _, recs = sim.resolve(2, 0, 8, [1])          # 1 is a miss again; evicts the LRU entry (key 0, slot 0)
    assert (recs[0].hit, recs[0].slot, recs[0].victim) == (0, 0, 0)
