"""Pins for the oracle's expert FFN, combine, int4 dequant and whole layer."""
import math

import numpy as np
import pytest

import oracle


def test_swiglu_scalar_closed_forms():
    # H = I = 1: y = silu(x*w1) * (x*w3) * w2 with silu(z) = z / (1 + e^-z)
    def ref(x, w1, w3, w2):
        g = x * w1
        return g / (1.0 + math.exp(-g)) * (x * w3) * w2
    for (x, w1, w3, w2) in [(1.0, 2.0, 3.0, 1.0), (1.0, 3.0, 2.0, 1.0), (-0.5, 1.5, 4.0, -2.0), (2.0, 0.0, 5.0, 1.0)]:
        y = oracle.swiglu_expert([[x]], [[w1]], [[w3]], [[w2]])[0, 0]
        assert abs(y - ref(x, w1, w3, w2)) < 1e-14
    # the gate is the x.W1 product: swapping W1 and W3 changes the answer
    a = oracle.swiglu_expert([[1.0]], [[2.0]], [[3.0]], [[1.0]])[0, 0]
    b = oracle.swiglu_expert([[1.0]], [[3.0]], [[2.0]], [[1.0]])[0, 0]
    assert abs(a - 6.0 / (1.0 + math.exp(-2.0))) < 1e-14
    assert abs(b - 6.0 / (1.0 + math.exp(-3.0))) < 1e-14


def test_swiglu_elementwise_rectangular():
    # H=3, I=2, M=2: every output element written out with the math module
    r = np.random.default_rng(0)
    X = r.standard_normal((2, 3))
    W1 = r.standard_normal((3, 2))
    W3 = r.standard_normal((3, 2))
    W2 = r.standard_normal((2, 3))
    y = oracle.swiglu_expert(X, W1, W3, W2)
    for m in range(2):
        h = []
        for i in range(2):
            g = math.fsum(X[m, c] * W1[c, i] for c in range(3))
            u = math.fsum(X[m, c] * W3[c, i] for c in range(3))
            h.append(g / (1.0 + math.exp(-g)) * u)
        for n in range(3):
            assert abs(y[m, n] - math.fsum(h[i] * W2[i, n] for i in range(2))) < 1e-13


def test_swiglu_linear_in_w2_and_w3():
    r = np.random.default_rng(1)
    X = r.standard_normal((4, 8))
    W1, W3 = r.standard_normal((8, 5)), r.standard_normal((8, 5))
    W2a, W2b = r.standard_normal((5, 8)), r.standard_normal((5, 8))
    ya = oracle.swiglu_expert(X, W1, W3, W2a)
    yb = oracle.swiglu_expert(X, W1, W3, W2b)
    assert np.allclose(oracle.swiglu_expert(X, W1, W3, W2a + 2 * W2b), ya + 2 * yb, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.swiglu_expert(X, W1, -3 * W3, W2a), -3 * ya, rtol=1e-12, atol=1e-12)
    assert np.all(oracle.swiglu_expert(X, np.zeros_like(W1), W3, W2a) == 0)  # silu(0) = 0


def _dense_reference(x, Wr, b, k, experts):
    """Every expert on every token, then masked by the routing: no permutation at all."""
    l = x @ Wr + b
    T, E = l.shape
    out = np.zeros((T, x.shape[1]))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l[t, e], e))[:k]
        z = np.array([math.exp(l[t, e] - l[t, order[0]]) for e in order])
        w = z / z.sum()
        for j, e in enumerate(order):
            g = x[t] @ experts[e][0]
            u = x[t] @ experts[e][1]
            out[t] += w[j] * (((g / (1 + np.exp(-g))) * u) @ experts[e][2])
    return out


@pytest.mark.parametrize("T,H,E,I,k", [(8, 16, 6, 12, 2), (13, 24, 9, 8, 3), (4, 8, 5, 6, 5)])
def test_layer_against_dense_all_experts(T, H, E, I, k):
    r = np.random.default_rng(T + H + E)
    x = r.standard_normal((T, H))
    Wr = r.standard_normal((H, E)) / math.sqrt(H)
    b = r.standard_normal(E) * 0.3
    experts = [(r.standard_normal((H, I)), r.standard_normal((H, I)), r.standard_normal((I, H))) for _ in range(E)]
    res = oracle.moe_layer(x, Wr, b, k, lambda e: experts[e])
    ref = _dense_reference(x, Wr, b, k, experts)
    assert np.allclose(res["out"], ref, rtol=1e-11, atol=1e-11)


def test_identical_experts_routing_independent():
    r = np.random.default_rng(7)
    T, H, E, I = 10, 12, 8, 6
    x = r.standard_normal((T, H))
    ex = (r.standard_normal((H, I)), r.standard_normal((H, I)), r.standard_normal((I, H)))
    single = oracle.swiglu_expert(x, *ex)
    for seed in range(3):
        Wr = np.random.default_rng(seed).standard_normal((H, E))
        out = oracle.moe_layer(x, Wr, None, 3, lambda e: ex)["out"]
        assert np.allclose(out, single, rtol=1e-12, atol=1e-12)


def test_k1_one_expert_is_plain_mlp():
    r = np.random.default_rng(8)
    x = r.standard_normal((5, 6))
    ex = (r.standard_normal((6, 4)), r.standard_normal((6, 4)), r.standard_normal((4, 6)))
    out = oracle.moe_layer(x, r.standard_normal((6, 1)), None, 1, lambda e: ex)["out"]
    assert np.allclose(out, oracle.swiglu_expert(x, *ex), rtol=0, atol=1e-14)


def test_combine_identical_rows_and_weights():
    y = np.tile(np.arange(5.0), (6, 1))
    perm_pos = np.array([[0, 1, 2], [3, 4, 5]])
    w = np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]])
    assert np.allclose(oracle.combine(y, perm_pos, w), np.tile(np.arange(5.0), (2, 1)), atol=1e-15)
    # one-hot weights pick the row
    y2 = np.arange(12.0).reshape(6, 2)
    out = oracle.combine(y2, perm_pos, np.array([[0, 1.0, 0], [0, 0, 1.0]]))
    assert out.tolist() == [[2.0, 3.0], [10.0, 11.0]]


def test_dequant_int4_groups():
    K, N, g = 256, 3, 128
    q = np.zeros((K, N), dtype=np.int8)
    q[0, 0], q[127, 0], q[128, 0], q[255, 2] = 7, -7, 1, -3
    s = np.array([[0.5, 1.0, 2.0], [0.25, 4.0, 8.0]], dtype=np.float16)
    W = oracle.dequant_int4(q, s, g)
    assert W[0, 0] == 3.5 and W[127, 0] == -3.5 and W[128, 0] == 0.25 and W[255, 2] == -24.0
    assert np.count_nonzero(W) == 4


def test_int4_quantiser_roundtrip_bound():
    # harness quantiser + oracle dequant: |W - q*s| <= s/2 per element, and s = fp16(max/7)
    import torch
    from workloads.gen import quantize_int4
    w = torch.randn(256, 8, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    q, s = quantize_int4(w, 128)
    assert int(q.abs().max()) <= 7
    Wd = oracle.dequant_int4(q, s, 128)
    wf = w.double().numpy()
    sf = np.repeat(s.double().numpy(), 128, axis=0)
    assert np.all(np.abs(wf - Wd) <= sf / 2 * (1 + 1e-3) + 1e-12)
