"""Comparison rules between the HIP path and the oracle.

  * top-k: the selected sets must be identical for every token that the
    oracle does not flag (k-th/(k+1)-th fp64 logit gap below 1e-4);
  * everything downstream of the selection (weights, permutation, cache
    trace, outputs) is compared against the oracle re-run on the GPU's own
    selection, so a legitimately different choice on a flagged token does not
    cascade;
  * integer results bit-exact; floating point within rel-L2 <= 1e-2 and
    max-abs <= 5e-2 * RMS(reference).
"""
import numpy as np

import oracle

REL_L2 = 1e-2
MAX_ABS_RMS = 5e-2
W_ATOL = 1e-5
FLAG_GAP = 1e-4


def np64(t):
    return oracle.moe.as_f64(t)


def npi(t):
    return t.detach().cpu().numpy().astype(np.int64)


def check_close(got, ref, what="", rel_l2=REL_L2, max_abs_rms=MAX_ABS_RMS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / nref if nref > 0 else err
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    mx = np.max(np.abs(got - ref)) if ref.size else 0.0
    assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e} > {rel_l2}"
    assert mx <= max_abs_rms * rms + 1e-30, f"{what}: max-abs {mx:.3e} > {max_abs_rms}*RMS={max_abs_rms * rms:.3e}"
    return rel, mx


def check_routing(gpu_idx, gpu_w, logits64, k):
    """Sets equal on unflagged tokens; GPU weights match the fp64 softmax over the GPU's own set."""
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    T, E = logits64.shape
    assert gpu_idx.shape == (T, k), f"selection shape {gpu_idx.shape} != {(T, k)}"
    assert np.all((gpu_idx >= 0) & (gpu_idx < E)), "expert index out of range"
    if T:
        srt = np.sort(gpu_idx, axis=1)
        assert np.all(np.diff(srt, axis=1) > 0), "a token selected the same expert twice"
    ref_idx = oracle.topk_select(logits64, k)
    flags = oracle.topk_flags(logits64, k)
    same = np.array([set(a) == set(b) for a, b in zip(gpu_idx.tolist(), ref_idx.tolist())], dtype=bool)
    bad = np.nonzero(~same & ~flags)[0]
    assert len(bad) == 0, f"top-k sets differ on {len(bad)} unflagged tokens, e.g. {bad[:5]}"
    # a differing set on a flagged token must still be a top-k up to the flag's gap: every chosen logit at least
    # every unchosen one minus the gap
    for t in np.nonzero(~same)[0]:
        chosen = np.zeros(E, dtype=bool)
        chosen[gpu_idx[t]] = True
        lo = logits64[t, chosen].min()
        hi = logits64[t, ~chosen].max() if k < E else -np.inf
        assert lo >= hi - FLAG_GAP, f"token {t}: selection is not a top-{k} (chosen min {lo}, unchosen max {hi})"
    # weights of the GPU's selection, in its order, from fp64 logits
    w_ref = oracle.topk_weights(logits64, gpu_idx)
    dw = np.max(np.abs(np.asarray(gpu_w, dtype=np.float64) - w_ref)) if gpu_w.size else 0.0
    assert dw <= W_ATOL, f"combine weights differ by {dw:.3e}"
    # the GPU's order must be by non-increasing fp64 logit up to rounding
    sel = np.take_along_axis(logits64, gpu_idx, axis=1)
    assert np.all(np.diff(sel, axis=1) <= 1e-4)
    return flags, same


def check_permutation(gpu_idx, counts, offsets, perm_src, perm_pos, E):
    c, o, pp, ps = oracle.permute(np.asarray(gpu_idx), E)
    assert np.array_equal(np.asarray(counts), c), "counts differ"
    assert np.array_equal(np.asarray(offsets), o), "offsets differ"
    assert np.array_equal(np.asarray(perm_pos), pp), "perm_pos differs"
    assert np.array_equal(np.asarray(perm_src)[:len(ps)], ps), "perm_src differs"
    return c, o, pp, ps
