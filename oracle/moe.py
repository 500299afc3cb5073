"""Plain fp64 statement of the routed expert layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never does.

What the pages fix (page "FreeToken-rtx-4090", section "How the MoE Memory
Hierarchy Works"): each token activates a small subset of the routed experts
of a layer -- six of 256 in the model the page describes -- and an expert is
executed as one complete unit wherever it resides. Caching and copying decide
where an expert's weights are read from, never what is computed, so this
oracle is the plain layer and ignores placement entirely.

What the pages leave open, and the reading taken here (the plainest standard
one for a routed mixture-of-experts layer):
  * router: a linear gate, l = x.Wr + b, with the bias added before selection
    and before the softmax;
  * selection: the k largest logits, in descending order, ties to the lower
    expert index, -0 equal to +0;
  * weights: softmax over all experts renormalised over the selected k, which
    equals a softmax over the k selected logits;
  * permutation: rows grouped by expert in ascending order, tokens in ascending
    order inside a group;
  * expert: SwiGLU, y = (silu(x.W1) * (x.W3)).W2 with W1, W3 [H, I], W2 [I, H];
  * combine: out_t = sum_j w_tj * y_tj;
  * int4 experts: W = q * s, q in [-7, 7], one fp16 scale per 128 rows of K and
    output column;
  * MXFP4 experts (the format's name is all the pages give): the OCP MX FP4
    format, W = E2M1(code) * 2^(scale - 127), one 8-bit scale per 32 rows of K
    and output column; activations stay bf16.
Every value is computed in fp64 from the exact values the layer is given.
"""
import numpy as np


def as_f64(a):
    """Exact fp64 copy of an array or a (CPU or device) torch tensor."""
    if hasattr(a, "detach"):  # torch tensor, converted without importing torch here
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def as_int(a):
    if hasattr(a, "detach"):
        return a.detach().cpu().numpy().astype(np.int64)
    return np.asarray(a, dtype=np.int64)


def router_logits(x, Wr, b=None):
    """Gate logits l[t, e] = sum_h x[t, h] * Wr[h, e] + b[e], in fp64."""
    x = as_f64(x)
    Wr = as_f64(Wr)
    l = x @ Wr
    if b is not None:
        l = l + as_f64(b)[None, :]
    return l


def topk_select(l, k):
    """Indices of the k largest logits per token, largest first.

    Built by k rounds of "take the largest remaining value"; np.argmax returns
    the first maximal position, so equal values go to the lower expert index,
    and it compares -0.0 and +0.0 as equal.
    """
    l = np.asarray(l, dtype=np.float64)
    T, E = l.shape
    assert 1 <= k <= E
    out = np.empty((T, k), dtype=np.int64)
    work = l.copy()
    rows = np.arange(T)
    for j in range(k):
        a = np.argmax(work, axis=1)
        out[:, j] = a
        work[rows, a] = -np.inf
    return out


def topk_flags(l, k, gap=1e-4):
    """True for tokens whose k-th and (k+1)-th largest logits differ by less than `gap`.

    Such tokens may legitimately select a different set under another
    summation order. With k == E nothing can differ, so nothing is flagged.
    """
    l = np.asarray(l, dtype=np.float64)
    T, E = l.shape
    if k >= E:
        return np.zeros(T, dtype=bool)
    v = -np.sort(-l, axis=1)
    return (v[:, k - 1] - v[:, k]) < gap


def topk_weights(l, idx):
    """Combine weights w[t, j] = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the selected logits."""
    l = np.asarray(l, dtype=np.float64)
    sel = np.take_along_axis(l, np.asarray(idx), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def permute(idx, E):
    """Group the (token, slot) pairs by expert.

    Returns counts [E], offsets [E+1] (exclusive prefix sum of counts),
    perm_pos [T, k] (row of pair (t, j) in expert order) and perm_src [T*k]
    (token of each row). Rows are ordered by expert, then by token, by
    handing out each expert's rows in token order.
    """
    idx = as_int(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:-1].copy()
    perm_pos = np.empty((T, k), dtype=np.int64)
    perm_src = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            perm_pos[t, j] = nxt[e]
            perm_src[nxt[e]] = t
            nxt[e] += 1
    return counts, offsets, perm_pos, perm_src


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(X, W1, W3, W2):
    """One expert on rows X [M, H]: y = (silu(X.W1) * (X.W3)).W2, fp64."""
    X = as_f64(X)
    g = X @ as_f64(W1)
    u = X @ as_f64(W3)
    h = silu(g) * u
    return h @ as_f64(W2)


def dequant_int4(q, s, group=128):
    """W[k, n] = q[k, n] * s[k // group, n] (exact in fp64)."""
    q = as_f64(q)
    s = as_f64(s)
    K, N = q.shape
    return (q.reshape(K // group, group, N) * s[:, None, :]).reshape(K, N)


def e2m1_value(code):
    """Value of a 4-bit FP4 (E2M1) code, from its fields: bit 3 sign, bits 2..1
    exponent (bias 1), bit 0 mantissa; exponent 0 is subnormal (m * 2^-1).
    OCP Microscaling Formats (MX) v1.0, the FP4 element format. The pages give
    the format's name only (page "FreeToken-benchmark", model table, the
    DeepSeek-V4-Flash row: routed experts in MXFP4)."""
    code = int(code)
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(s):
    """Value of an 8-bit E8M0 block scale: 2^(s - 127); 255 is NaN (same standard)."""
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def dequant_mxfp4(codes, scales, block=32):
    """W[k, n] = E2M1[codes[k, n]] * 2^(scales[k // block, n] - 127): one scale per
    `block` consecutive K values of a column (exact in fp64)."""
    c = codes.detach().cpu().numpy() if hasattr(codes, "detach") else np.asarray(codes)
    K, N = c.shape
    w = E2M1[c].reshape(K // block, block, N)
    w *= e8m0_value(as_int(scales))[:, None, :]
    return w.reshape(K, N)


def expert_outputs(x, offsets, perm_src, get_expert, experts=None):
    """y_perm [T*k, H]: row r holds expert e's output for token perm_src[r].

    `get_expert(e)` returns (W1, W3, W2) of expert e. Only experts listed in
    `experts` (default: every expert with rows) are evaluated.
    """
    x = as_f64(x)
    offsets = as_int(offsets)
    perm_src = as_int(perm_src)
    E = len(offsets) - 1
    y = np.zeros((len(perm_src), x.shape[1]), dtype=np.float64)
    for e in (range(E) if experts is None else experts):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            y[a:b] = swiglu_expert(x[perm_src[a:b]], *get_expert(e))
    return y


def combine(y_perm, perm_pos, w):
    """out[t] = sum_j w[t, j] * y_perm[perm_pos[t, j]], j ascending."""
    y_perm = np.asarray(y_perm, dtype=np.float64)
    perm_pos = as_int(perm_pos)
    w = np.asarray(w, dtype=np.float64)
    T, k = perm_pos.shape
    out = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y_perm[perm_pos[:, j]]
    return out


def moe_layer(x, Wr, b, k, get_expert):
    """The whole layer on one batch; returns every intermediate as a dict."""
    l = router_logits(x, Wr, b)
    E = l.shape[1]
    idx = topk_select(l, k)
    w = topk_weights(l, idx)
    counts, offsets, perm_pos, perm_src = permute(idx, E)
    y_perm = expert_outputs(x, offsets, perm_src, get_expert)
    out = combine(y_perm, perm_pos, w)
    return dict(logits=l, idx=idx, w=w, flags=topk_flags(l, k), counts=counts, offsets=offsets,
                perm_pos=perm_pos, perm_src=perm_src, y_perm=y_perm, out=out)
