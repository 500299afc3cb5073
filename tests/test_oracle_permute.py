"""Pins for the oracle's permutation (counts, offsets, perm_pos, perm_src)."""
import numpy as np
import pytest

import oracle


def routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    return np.stack([r.permutation(E)[:k] for _ in range(T)])


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (8, 16, 2), (37, 16, 5), (300, 64, 6), (5, 6, 6)])
def test_permute_against_stable_sort(T, E, k):
    idx = routing(T, E, k, T * 7 + E)
    counts, offsets, perm_pos, perm_src = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    # library stable sort of the flattened (t, j) pairs by expert: ties keep (t, j) order
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(perm_src, order // k)
    inv = np.empty_like(order)
    inv[order] = np.arange(T * k)
    assert np.array_equal(perm_pos.reshape(-1), inv)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * k


def test_permute_invariants():
    T, E, k = 64, 32, 8
    idx = routing(T, E, k, 11)
    counts, offsets, perm_pos, perm_src = oracle.permute(idx, E)
    # perm_src[perm_pos[t, j]] == t  (unpermute . permute = identity)
    for t in range(T):
        for j in range(k):
            assert perm_src[perm_pos[t, j]] == t
    # each row lands in its expert's segment, tokens ascending inside a segment
    for e in range(E):
        seg = perm_src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert all(e in idx[t] for t in seg)
    # positions are a permutation of 0..T*k-1
    assert sorted(perm_pos.reshape(-1).tolist()) == list(range(T * k))


def test_permute_degenerate():
    # every token picks the same experts (k == E): rows are token order in each segment
    T, E = 5, 3
    idx = np.tile(np.array([2, 0, 1]), (T, 1))
    counts, offsets, perm_pos, perm_src = oracle.permute(idx, E)
    assert counts.tolist() == [5, 5, 5]
    assert perm_src.tolist() == [0, 1, 2, 3, 4] * 3
    assert perm_pos[:, 0].tolist() == [10, 11, 12, 13, 14]
