"""GPU parity of each kernel stage against the oracle, with the oracle's inputs
injected per stage (routing, grouped FFN, combine) at sizes the oracle checks
element by element: several tiles plus ragged tails, empty groups, k = 1 and
k = E, every weight format.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.parity import check_close, check_permutation, check_routing, np64, npi
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu

dev = "cuda"


@pytest.fixture(scope="module")
def L():
    from routed_expert_layer_amd import _lib
    return _lib


def cfg_like(base, **kw):
    return dataclasses.replace(CONFIGS[base], **kw)


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------
ROUTE_CASES = [
    # name, base config, overrides
    ("tiny_f32", "tiny_f32_h256_e16", {}),
    ("decode_bf16_t1", "decode_bf16_h4096_e256", {}),
    ("stack_bf16_t4", "stack48_bf16_h2048_e128", {}),
    ("ragged_bf16_t300", "decode_bf16_h4096_e256", dict(name="ragged300", T=300, H=512, E=64, k=6)),
    ("k1", "tiny_f32_h256_e16", dict(name="k1", T=77, k=1)),
    ("k_eq_e", "tiny_f32_h256_e16", dict(name="kE", T=70, E=8, k=8)),
    ("e_not_mult64_bf16", "decode_bf16_h4096_e256", dict(name="e100", T=130, H=256, E=100, k=5, zipf_s=1.5)),
    ("t0", "tiny_f32_h256_e16", dict(name="t0", T=0)),
    ("small_t16_e512", "decode_bf16_h4096_e256", dict(name="s16", T=16, H=256, E=512, k=8)),
    ("gemm_router_t300", "decode_bf16_h4096_e256", dict(name="g300", T=300, H=512, E=256, k=6, zipf_s=0.0)),
    ("gemm_router_t1000", "decode_bf16_h4096_e256", dict(name="g1000", T=1000, H=1024, E=128, k=8, zipf_s=1.5)),
]


@pytest.mark.parametrize("name,base,kw", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_parity(L, name, base, kw):
    from routed_expert_layer_amd.runtime import RouteBuffers
    cfg = cfg_like(base, **kw)
    print(f"route case {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} {cfg.act}", flush=True)
    rb = RouteBuffers(max(cfg.T, 1), cfg.H, cfg.E, cfg.k, dev, keep_logits=True)
    Wr = gen.router_weight(cfg, 0, dev)
    steps = 4 if cfg.T > 1 else 16
    for step in range(steps):
        b = gen.router_bias(cfg, 0, step, dev)
        x = gen.tokens(cfg, step, 0, dev)
        rb.route(x, Wr, b)
        torch.cuda.synchronize()
        T = cfg.T
        counts = npi(rb.counts)
        offsets = npi(rb.offsets)
        if T == 0:
            assert counts.sum() == 0 and np.all(offsets == 0)
            continue
        l64 = oracle.router_logits(x, Wr, b)
        check_close(np64(rb.logits[:T]), l64, "logits", rel_l2=1e-5, max_abs_rms=1e-4)
        idx = npi(rb.topk_idx[:T])
        check_routing(idx, np64(rb.topk_w[:T]), l64, cfg.k)
        check_permutation(idx, counts, offsets, npi(rb.perm_src[:T * cfg.k]), npi(rb.perm_pos[:T]), cfg.E)


def test_route_ties_and_signed_zero(L):
    """Exact ties (all-zero gate) go to the lower expert index; -0 equals +0."""
    from routed_expert_layer_amd.runtime import RouteBuffers
    T, H, E, k = 65, 64, 20, 4
    rb = RouteBuffers(T, H, E, k, dev, keep_logits=True)
    x = torch.zeros((T, H), dtype=torch.float32, device=dev)
    Wr = torch.zeros((H, E), dtype=torch.float32, device=dev)
    b = torch.zeros(E, dtype=torch.float32, device=dev)
    b[5] = -0.0
    b[7] = 1.0
    b[9] = 1.0
    rb.route(x, Wr, b)
    torch.cuda.synchronize()
    idx = npi(rb.topk_idx)
    assert np.all(idx == np.array([7, 9, 0, 1]))
    w = np64(rb.topk_w)
    e = np.exp(-1.0)
    assert np.allclose(w, np.array([1, 1, e, e]) / (2 + 2 * e), atol=1e-6)


# ---------------------------------------------------------------------------
# Grouped expert FFN (teacher-forced routing)
# ---------------------------------------------------------------------------
def _experts(cfg, n, wfmt):
    out = []
    for e in range(n):
        if wfmt == "int4":
            out.append(gen.expert_int4(cfg, 0, e, dev))
        elif wfmt == "mxfp4":
            out.append(gen.expert_mxfp4(cfg, 0, e, dev))
        else:
            out.append(gen.expert_weights(cfg, 0, e, dev))
    return out


def _canon64(w, wfmt, group=128):
    if wfmt == "int4":
        return (oracle.dequant_int4(w["q1"], w["s1"], group), oracle.dequant_int4(w["q3"], w["s3"], group),
                oracle.dequant_int4(w["q2"], w["s2"], group))
    if wfmt == "mxfp4":
        return (oracle.dequant_mxfp4(w["c1"], w["s1"]), oracle.dequant_mxfp4(w["c3"], w["s3"]),
                oracle.dequant_mxfp4(w["c2"], w["s2"]))
    return tuple(np64(t) for t in w)


FFN_CASES = [
    # name, wfmt, H, I, rows per expert, mode
    ("f32_tiny", "f32", 256, 128, [3, 0, 1, 8, 2], "auto"),
    ("bf16_decode", "bf16", 512, 256, [1, 0, 6, 16, 17, 2, 33], "decode"),
    ("bf16_decode_k_odd", "bf16", 384, 160, [5, 1, 0, 9], "decode"),
    ("bf16_prefill", "bf16", 512, 256, [130, 0, 1, 127, 128, 300, 17, 777], "prefill"),
    ("bf16_prefill_c3shape", "bf16", 2048, 768, [70, 3, 129], "prefill"),
    # partial last tiles whose waves hold 1, 2, 3 or 4 token fragments of the group (the GEMMs run a K loop
    # per count): 128-token tiles for 40, 110, 200 rows, 256-token tiles for 276 and 356 rows
    ("bf16_prefill_partial", "bf16", 512, 256, [40, 110, 276, 356, 200], "prefill"),
    ("int4_decode", "int4", 512, 256, [1, 8, 0, 3, 20], "decode"),
    ("int4_decode_wide", "int4", 1024, 384, [2, 16, 5], "decode"),
    ("mxfp4_decode", "mxfp4", 512, 256, [1, 8, 0, 3, 20], "decode"),
    ("mxfp4_decode_wide", "mxfp4", 1024, 384, [2, 16, 5, 33], "decode"),
    ("mxfp4_prefill", "mxfp4", 512, 256, [130, 0, 1, 127, 128, 300, 17, 777], "prefill"),
    ("mxfp4_prefill_c3shape", "mxfp4", 2048, 768, [70, 3, 129], "prefill"),
    ("mxfp4_prefill_partial", "mxfp4", 512, 256, [40, 110, 276, 356, 200], "prefill"),
    ("mxfp4_auto_mixed", "mxfp4", 512, 384, [40, 2, 250], "auto"),
]


@pytest.mark.parametrize("name,wfmt,H,I,rows,mode", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_ffn_parity(L, name, wfmt, H, I, rows, mode):
    print(f"ffn case {name}: {wfmt} H={H} I={I} rows={rows} mode={mode}", flush=True)
    act = "f32" if wfmt == "f32" else "bf16"
    cfg = cfg_like("tiny_f32_h256_e16", name=f"ffn_{name}", H=H, I=I, E=len(rows), act=act, wfmt=wfmt)
    E = len(rows)
    T = max(40, max(rows))
    x = gen.tokens(cfg, 0, 0, dev, T=T)
    r = np.random.default_rng(len(name))
    perm_src = np.concatenate([r.integers(0, T, size=n) for n in rows]).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    wf = {"f32": L.MOE_W_F32, "bf16": L.MOE_W_BF16, "int4": L.MOE_W_INT4, "mxfp4": L.MOE_W_MXFP4}[wfmt]
    blob = L.moe_expert_bytes(wf, H, I)
    stride = (blob + 4095) // 4096 * 4096
    slot_of = [(e + 1) % E for e in range(E)]  # non-identity slot mapping
    slots = torch.zeros(E * stride, dtype=torch.uint8, device=dev)
    ex = _experts(cfg, E, wfmt)
    for e in range(E):
        w = ex[e]
        dst = slots[slot_of[e] * stride:]
        if wfmt == "int4":
            L.moe_pack_expert(wf, H, I, w["q1"], w["q3"], w["q2"], w["s1"], w["s3"], w["s2"], dst)
        elif wfmt == "mxfp4":
            L.moe_pack_expert(wf, H, I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"], dst)
        else:
            L.moe_pack_expert(wf, H, I, w[0], w[1], w[2], None, None, None, dst)
    work = np.array([[e, slot_of[e], off[e], rows[e]] for e in range(E)], dtype=np.int32)
    rows_total = int(off[-1])
    y = torch.full((rows_total, H), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(L.moe_ffn_workspace_size(rows_total, H, I, wf), dtype=torch.uint8, device=dev)
    ps = torch.from_numpy(perm_src).to(dev)
    m = {"auto": L.MOE_FFN_AUTO, "decode": L.MOE_FFN_DECODE, "prefill": L.MOE_FFN_PREFILL}[mode]
    L.moe_ffn(x, ps, work, slots, stride, wf, H, I, y, ws, m)
    torch.cuda.synchronize()
    yg = np64(y)
    x64 = np64(x)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b == a:
            continue
        ref = oracle.swiglu_expert(x64[perm_src[a:b]], *_canon64(ex[e], wfmt))
        check_close(yg[a:b], ref, f"{name} expert {e}")


@pytest.mark.gpu
@pytest.mark.parametrize("wfmt", ["bf16", "int4", "mxfp4"])
def test_ffn_decode_large_activations(L, wfmt):
    """Activations 4096 times the usual scale (exact in bf16: a power of two), so that the gate/up sums and the
    SwiGLU product reach ~1e7, far past the fp16 range: the decode kernels keep them in bf16 / fp32 and still
    match the oracle."""
    H, I, rows = 512, 256, [1, 8, 3]
    cfg = cfg_like("tiny_f32_h256_e16", name=f"ffn_large_{wfmt}", H=H, I=I, E=len(rows), act="bf16", wfmt=wfmt)
    E, T = len(rows), 12
    x = (gen.tokens(cfg, 0, 0, dev, T=T).float() * 4096.0).to(torch.bfloat16)
    r = np.random.default_rng(7)
    perm_src = np.concatenate([r.integers(0, T, size=n) for n in rows]).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    wf = {"bf16": L.MOE_W_BF16, "int4": L.MOE_W_INT4, "mxfp4": L.MOE_W_MXFP4}[wfmt]
    stride = (L.moe_expert_bytes(wf, H, I) + 4095) // 4096 * 4096
    slots = torch.zeros(E * stride, dtype=torch.uint8, device=dev)
    ex = _experts(cfg, E, wfmt)
    for e in range(E):
        w, dst = ex[e], slots[e * stride:]
        if wfmt == "int4":
            L.moe_pack_expert(wf, H, I, w["q1"], w["q3"], w["q2"], w["s1"], w["s3"], w["s2"], dst)
        elif wfmt == "mxfp4":
            L.moe_pack_expert(wf, H, I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"], dst)
        else:
            L.moe_pack_expert(wf, H, I, w[0], w[1], w[2], None, None, None, dst)
    work = np.array([[e, e, off[e], rows[e]] for e in range(E)], dtype=np.int32)
    y = torch.full((int(off[-1]), H), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(L.moe_ffn_workspace_size(int(off[-1]), H, I, wf), dtype=torch.uint8, device=dev)
    L.moe_ffn(x, torch.from_numpy(perm_src).to(dev), work, slots, stride, wf, H, I, y, ws, L.MOE_FFN_DECODE)
    torch.cuda.synchronize()
    yg, x64 = np64(y), np64(x)
    assert np.isfinite(yg).all()
    for e in range(E):
        a, b = off[e], off[e + 1]
        ref = oracle.swiglu_expert(x64[perm_src[a:b]], *_canon64(ex[e], wfmt))
        assert np.abs(ref).max() > 1e6  # the range fp16 could not hold
        check_close(yg[a:b], ref, f"large activations {wfmt} expert {e}")


GROUPED_CASES = [
    # name, wfmt, H, I, rows per expert (seeded random when an int: that many experts of 0..maxrows rows)
    ("bf16_ragged", "bf16", 512, 256, [130, 0, 1, 127, 128, 300, 17, 777, 256, 257, 40, 110, 276, 356, 200]),
    ("bf16_many_rounds", "bf16", 256, 128, (200, 300)),
    ("bf16_1000_experts", "bf16", 256, 128, (1000, 6)),
    ("bf16_c3shape", "bf16", 2048, 768, [70, 3, 129, 513]),
    ("mxfp4_ragged", "mxfp4", 512, 256, [130, 0, 1, 127, 128, 300, 17, 777, 40, 110, 276]),
    ("mxfp4_many_rounds", "mxfp4", 256, 128, (120, 300)),
]


@pytest.mark.parametrize("name,wfmt,H,I,rows", GROUPED_CASES, ids=[c[0] for c in GROUPED_CASES])
def test_grouped_ffn_parity(L, name, wfmt, H, I, rows):
    """moe_ffn_grouped (work list planned on the GPU from device counts and offsets, GEMM blocks looping over
    super-tiles) against the oracle per group; bit-identical to moe_ffn's host-planned GEMM on the same groups;
    a group whose slot is out of range and a group reaching past rows_max are left untouched."""
    if isinstance(rows, tuple):
        n, mx = rows
        rows = [int(v) for v in np.random.default_rng(n + mx).integers(0, mx + 1, size=n)]
    E = len(rows)
    print(f"grouped ffn case {name}: {wfmt} H={H} I={I} E={E} rows={sum(rows)}", flush=True)
    cfg = cfg_like("tiny_f32_h256_e16", name=f"grp_{name}", H=H, I=I, E=E, act="bf16", wfmt=wfmt)
    T = max(40, max(rows))
    x = gen.tokens(cfg, 0, 0, dev, T=T)
    r = np.random.default_rng(len(name) + E)
    perm_src = np.concatenate([r.integers(0, T, size=n) for n in rows]).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    wf = L.MOE_W_MXFP4 if wfmt == "mxfp4" else L.MOE_W_BF16
    stride = (L.moe_expert_bytes(wf, H, I) + 4095) // 4096 * 4096
    slot_of = np.array([(e + 3) % E for e in range(E)], np.int32)  # non-identity slot mapping
    nonempty = [e for e in range(E) if rows[e] > 0]
    bad_slot = nonempty[len(nonempty) // 2]  # this group's slot is out of range: skipped
    slot_of[bad_slot] = E
    rows_total = int(off[-1])
    last = nonempty[-1]
    rows_max = rows_total - 1  # the last group reaches past rows_max: skipped
    slots = torch.zeros(E * stride, dtype=torch.uint8, device=dev)
    ex = {}
    for e in nonempty:
        w = gen.expert_mxfp4(cfg, 0, e, dev) if wfmt == "mxfp4" else gen.expert_weights(cfg, 0, e, dev)
        ex[e] = w
        if slot_of[e] >= E:
            continue
        dst = slots[int(slot_of[e]) * stride:]
        if wfmt == "mxfp4":
            L.moe_pack_expert(wf, H, I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"], dst)
        else:
            L.moe_pack_expert(wf, H, I, w[0], w[1], w[2], None, None, None, dst)
    y = torch.full((rows_total, H), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(L.moe_ffn_workspace_size(rows_total, H, I, wf), dtype=torch.uint8, device=dev)
    ps = torch.from_numpy(perm_src).to(dev)
    counts_d = torch.tensor(rows, dtype=torch.int32, device=dev)
    off_d = torch.from_numpy(off.astype(np.int32)).to(dev)
    L.moe_ffn_grouped(x, ps, counts_d, off_d, torch.from_numpy(slot_of).to(dev), E, rows_max, slots, stride, wf,
                      H, I, y, ws)
    torch.cuda.synchronize()
    yg = np64(y)
    x64 = np64(x)
    for e in nonempty:
        a, b = off[e], off[e + 1]
        if e in (bad_slot, last):
            assert np.all(np.isnan(yg[a:b])), f"{name}: skipped group {e} was written"
            continue
        ref = oracle.swiglu_expert(x64[perm_src[a:b]], *_canon64(ex[e], wfmt))
        check_close(yg[a:b], ref, f"{name} expert {e}")
    # the host-planned GEMM on the same groups gives the same bits
    work = np.array([[e, slot_of[e], off[e], rows[e]] for e in nonempty if e not in (bad_slot, last)], np.int32)
    y2 = torch.full((rows_total, H), float("nan"), dtype=torch.float32, device=dev)
    ws2 = torch.empty(L.moe_ffn_workspace_size(rows_total, H, I, wf), dtype=torch.uint8, device=dev)
    L.moe_ffn(x, ps, work, slots, stride, wf, H, I, y2, ws2, L.MOE_FFN_PREFILL)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(y, nan=7.0), torch.nan_to_num(y2, nan=7.0)), \
        f"{name}: device-planned and host-planned GEMMs differ"


@pytest.mark.parametrize("wfmt", ["bf16", "mxfp4"])
def test_clock_record_leaves_prefill_unchanged(L, wfmt):
    # the clock diagnostic only adds counters: the GEMM output is bit-identical with it on, the counters
    # give a plausible shader clock, and once it is off they stay as they are
    print(f"clock record case: {wfmt}", flush=True)
    H, I, rows = 512, 256, [130, 0, 300, 17]
    E = len(rows)
    cfg = cfg_like("tiny_f32_h256_e16", name=f"clk_{wfmt}", H=H, I=I, E=E, act="bf16", wfmt=wfmt)
    T = max(rows)
    x = gen.tokens(cfg, 0, 0, dev, T=T)
    r = np.random.default_rng(7)
    perm_src = torch.from_numpy(np.concatenate([r.integers(0, T, size=n) for n in rows]).astype(np.int32)).to(dev)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    wf = L.MOE_W_MXFP4 if wfmt == "mxfp4" else L.MOE_W_BF16
    stride = (L.moe_expert_bytes(wf, H, I) + 4095) // 4096 * 4096
    slots = torch.zeros(E * stride, dtype=torch.uint8, device=dev)
    for e, w in enumerate(_experts(cfg, E, wfmt)):
        if wfmt == "mxfp4":
            L.moe_pack_expert(wf, H, I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"], slots[e * stride:])
        else:
            L.moe_pack_expert(wf, H, I, w[0], w[1], w[2], None, None, None, slots[e * stride:])
    work = np.array([[e, e, off[e], rows[e]] for e in range(E)], dtype=np.int32)
    n = int(off[-1])
    ws = torch.empty(L.moe_ffn_workspace_size(n, H, I, wf), dtype=torch.uint8, device=dev)
    ys = []
    sums = torch.zeros(2, dtype=torch.int64, device=dev)
    for record in (False, True, False):
        y = torch.full((n, H), float("nan"), dtype=torch.float32, device=dev)
        L.moe_clock_record(sums if record else None)
        try:
            L.moe_ffn(x, perm_src, work, slots, stride, wf, H, I, y, ws, L.MOE_FFN_PREFILL)
            torch.cuda.synchronize()
        finally:
            L.moe_clock_record(None)
        ys.append(y)
        if record:
            cyc, ticks = (int(v) for v in sums.cpu())
            assert cyc > 0 and ticks > 0
            assert 0.3 < cyc / ticks / 10.0 < 3.5, (cyc, ticks)
            after_on = (cyc, ticks)
    assert tuple(int(v) for v in sums.cpu()) == after_on
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


def test_ffn_zero_work_is_noop(L):
    y = torch.zeros((4, 256), dtype=torch.float32, device=dev)
    ws = torch.empty(1024, dtype=torch.uint8, device=dev)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=dev)
    L.moe_ffn(x, torch.zeros(4, dtype=torch.int32, device=dev), np.zeros((0, 4), np.int32), y, 1 << 20,
              L.MOE_W_BF16, 256, 128, y, ws)
    torch.cuda.synchronize()
    assert float(y.abs().sum()) == 0.0


# ---------------------------------------------------------------------------
# Combine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,H,out_bf16", [(1, 6, 4096, False), (37, 2, 256, False), (5, 3, 130, True)])
def test_combine_parity(L, T, k, H, out_bf16):
    g = torch.Generator(device=dev).manual_seed(T * 1000 + H)
    y = torch.randn((T * k, H), generator=g, device=dev)
    perm_pos = torch.randperm(T * k, generator=g, device=dev).to(torch.int32).reshape(T, k)
    w = torch.rand((T, k), generator=g, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16 if out_bf16 else torch.float32, device=dev)
    L.moe_combine(y, perm_pos, w, out)
    torch.cuda.synchronize()
    ref = oracle.combine(np64(y), npi(perm_pos), np64(w))
    if out_bf16:
        check_close(np64(out), ref, "combine bf16", rel_l2=4e-3)
    else:
        check_close(np64(out), ref, "combine", rel_l2=1e-6, max_abs_rms=1e-5)


@pytest.mark.gpu
def test_pack_matches_documented_layout(L):
    """The GPU packer writes, byte for byte, the blob layout the host expert kernel reads."""
    from tests.blob_layout import bf16_blob
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name="packlayout", H=512, I=384)
    W1, W3, W2 = gen.expert_weights(cfg, 0, 2, "cuda")
    blob = torch.empty(L.moe_expert_bytes(L.MOE_W_BF16, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    L.moe_pack_expert(L.MOE_W_BF16, cfg.H, cfg.I, W1, W3, W2, None, None, None, blob)
    torch.cuda.synchronize()
    ref = bf16_blob(W1.cpu(), W3.cpu(), W2.cpu())
    assert np.array_equal(blob.cpu().numpy().view(np.uint16), ref)


@pytest.mark.gpu
def test_pack_int4_matches_documented_layout(L):
    """The GPU packer writes the int4 blob layout the C ABI documents, byte for byte (padding aside)."""
    from tests.blob_layout import int4_blob
    cfg = dataclasses.replace(CONFIGS["decode_int4_t8_l8"], name="packi4", H=512, I=384, weights_of=None,
                              pool_layers=None)
    w = gen.expert_int4(cfg, 0, 3, "cuda")
    nb = L.moe_expert_bytes(L.MOE_W_INT4, cfg.H, cfg.I)
    blob = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    L.moe_pack_expert(L.MOE_W_INT4, cfg.H, cfg.I, w["q1"], w["q3"], w["q2"], w["s1"], w["s3"], w["s2"], blob)
    torch.cuda.synchronize()
    ref = int4_blob(*(w[k].cpu().numpy() for k in ("q1", "q3", "q2", "s1", "s3", "s2")))
    assert len(ref) == nb
    assert np.array_equal(blob.cpu().numpy(), ref)


@pytest.mark.gpu
def test_pack_mxfp4_matches_documented_layout(L):
    """The GPU packer writes the MXFP4 blob layout the C ABI documents, byte for byte (padding aside)."""
    from tests.blob_layout import mxfp4_blob
    cfg = dataclasses.replace(CONFIGS["decode_mxfp4_t8_l8"], name="packmx", H=512, I=384, weights_of=None,
                              pool_layers=None)
    w = gen.expert_mxfp4(cfg, 0, 3, "cuda")
    nb = L.moe_expert_bytes(L.MOE_W_MXFP4, cfg.H, cfg.I)
    blob = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    L.moe_pack_expert(L.MOE_W_MXFP4, cfg.H, cfg.I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"], blob)
    torch.cuda.synchronize()
    ref = mxfp4_blob(*(w[k].cpu().numpy() for k in ("c1", "c3", "c2", "s1", "s3", "s2")))
    assert len(ref) == nb
    assert np.array_equal(blob.cpu().numpy(), ref)
