"""Pins for the oracle's router, top-k selection, flags and combine weights.

Each check is independent of the oracle's own code path: a library sort, a
brute-force search over subsets, closed forms evaluated with the math module,
and special cases whose answer is known without computing.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def rng(seed=0):
    return np.random.default_rng(seed)


def test_logits_bruteforce_tiny():
    r = rng(1)
    x = r.standard_normal((3, 5))
    Wr = r.standard_normal((5, 4))
    b = r.standard_normal(4)
    l = oracle.router_logits(x, Wr, b)
    for t in range(3):
        for e in range(4):
            s = math.fsum(float(x[t, h]) * float(Wr[h, e]) for h in range(5)) + float(b[e])
            assert abs(l[t, e] - s) < 1e-12
    # a transposed operand would not even have this shape
    assert l.shape == (3, 4)


@pytest.mark.parametrize("k", [1, 2, 3, 6])
def test_topk_matches_stable_argsort(k):
    r = rng(2)
    l = np.round(r.standard_normal((200, 16)) * 2) / 2  # coarse grid: many exact ties
    idx = oracle.topk_select(l, k)
    ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref)


def test_topk_bruteforce_subsets():
    r = rng(3)
    E, k = 6, 3
    for _ in range(200):
        l = r.integers(-2, 3, size=E).astype(np.float64)  # heavy ties
        got = set(oracle.topk_select(l[None, :], k)[0].tolist())
        winners = []
        for S in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in S]
            # S is the top-k iff every member beats every non-member under (value desc, index asc)
            if all((l[a] > l[c]) or (l[a] == l[c] and a < c) for a in S for c in rest):
                winners.append(set(S))
        assert len(winners) == 1
        assert got == winners[0]


def test_topk_order_descending_and_ties_low_index():
    l = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert oracle.topk_select(l, 4)[0].tolist() == [1, 2, 4, 3]


def test_topk_special_cases():
    r = rng(4)
    # all logits equal -> experts 0..k-1
    assert oracle.topk_select(np.zeros((5, 8)), 3).tolist() == [[0, 1, 2]] * 5
    # a steep decreasing bias dominates any bounded gate
    E, k = 32, 6
    x = r.standard_normal((10, 16))
    Wr = r.standard_normal((16, E)) * 0.1
    b = -100.0 * np.arange(E)
    idx = oracle.topk_select(oracle.router_logits(x, Wr, b), k)
    assert idx.tolist() == [list(range(k))] * 10
    # -0.0 and +0.0 are equal: the lower index wins
    assert oracle.topk_select(np.array([[0.0, -0.0]]), 1)[0, 0] == 0
    assert oracle.topk_select(np.array([[-0.0, 0.0]]), 1)[0, 0] == 0


def test_flags():
    l = np.array([[3.0, 2.0, 2.0 - 5e-5, -1.0],    # gap 5e-5 < 1e-4 -> flagged
                  [3.0, 2.0, 2.0 - 2e-4, -1.0],    # gap 2e-4 -> not flagged
                  [3.0, 2.0, 2.0, -1.0]])          # exact tie at the boundary -> flagged
    assert oracle.topk_flags(l, 2).tolist() == [True, False, True]
    # a gap inside the selected set does not matter
    assert not oracle.topk_flags(np.array([[2.0, 2.0, -5.0]]), 2)[0]
    # k == E never flags
    assert not oracle.topk_flags(np.zeros((1, 4)), 4)[0]


def test_weights_closed_forms():
    r = rng(5)
    l = r.standard_normal((50, 12)) * 3
    for k in (1, 2, 6):
        idx = oracle.topk_select(l, k)
        w = oracle.topk_weights(l, idx)
        assert np.all(np.abs(w.sum(1) - 1.0) < 1e-12)
        assert np.all(np.diff(w, axis=1) <= 1e-15)  # descending logits -> non-increasing weights
        if k == 1:
            assert np.all(w == 1.0)
    # k == E equals the full softmax, evaluated term by term with math.exp
    idx = oracle.topk_select(l, 12)
    w = oracle.topk_weights(l, idx)
    for t in range(5):
        den = math.fsum(math.exp(v) for v in l[t])
        for j in range(12):
            assert abs(w[t, j] - math.exp(l[t, idx[t, j]]) / den) < 1e-13
    # equal logits -> 1/k
    w = oracle.topk_weights(np.zeros((2, 7)), oracle.topk_select(np.zeros((2, 7)), 4))
    assert np.allclose(w, 0.25, atol=0, rtol=1e-15)
    # two experts: w0 = sigmoid(l0 - l1)
    l2 = np.array([[0.7, -0.4, -3.0]])
    w2 = oracle.topk_weights(l2, oracle.topk_select(l2, 2))
    assert abs(w2[0, 0] - 1.0 / (1.0 + math.exp(-1.1))) < 1e-15
