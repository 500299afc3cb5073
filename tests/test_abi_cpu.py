"""C-ABI checks that need no GPU: exported symbols, argument validation and
error codes, and the host LRU policy (cache_resolve) against the oracle's
simulator, bit-exact. No compute call is made."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from routed_expert_layer_amd import _lib
    return _lib


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("if")))


def test_every_declared_symbol_is_exported(L):
    declared = header_functions()
    assert len(declared) >= 30
    lib = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, f"declared in include/moe.h but not exported: {missing}"
    assert sorted(L.SYMBOLS) == declared, "binding symbol list differs from the header"
    assert L.moe_abi_version() >= 1


def test_expert_bytes(L):
    assert L.moe_expert_bytes(L.MOE_W_BF16, 4096, 2048) == 3 * 4096 * 2048 * 2
    assert L.moe_expert_bytes(L.MOE_W_F32, 256, 128) == 3 * 256 * 128 * 4
    b = L.moe_expert_bytes(L.MOE_W_INT4, 4096, 2048)
    codes, scales = 3 * 4096 * 2048 // 2, 3 * 4096 * 2048 // 128 * 2
    assert codes + scales <= b < codes + scales + 4 * 256
    # unsupported shapes are rejected with size 0
    assert L.moe_expert_bytes(L.MOE_W_BF16, 100, 2048) == 0
    assert L.moe_expert_bytes(L.MOE_W_INT4, 4096, 200) == 0
    assert L.moe_expert_bytes(7, 64, 64) == 0


@pytest.mark.parametrize("S,E,Lyr,max_active,steps,split", [
    (8, 16, 1, 14, 64, None), (64, 256, 1, 6, 200, None), (16, 32, 6, 10, 40, None), (3, 12, 2, 9, 50, None),
    (1, 4, 1, 4, 30, None), (8, 16, 1, 14, 64, (1, 3)), (64, 256, 1, 6, 200, (56, 165)), (16, 32, 6, 10, 40, (2, 1)),
    (3, 12, 2, 9, 50, (0, 1)), (4, 16, 3, 8, 40, (5, 0))])
def test_cache_resolve_matches_oracle(L, S, E, Lyr, max_active, steps, split):
    r = np.random.default_rng(S + E + Lyr)
    cache = L.MoeCache(Lyr, E, S)
    sim = oracle.SharedLRU(S)
    if split:
        L.moe_cache_set_split(cache, *split)
        sim.set_split(*split)
    zipf = 1.0 / np.arange(1, E + 1) ** 1.2
    for step in range(steps):
        for layer in range(Lyr):
            n = int(r.integers(1, max_active + 1))
            ex = np.sort(r.choice(E, size=n, replace=False, p=zipf / zipf.sum())).astype(np.int32)
            we, wslot, wwave, misses, nw = L.cache_resolve(cache, step, layer, ex)
            waves, recs = sim.resolve(step, layer, E, ex)
            assert nw == len(waves)
            flat = [(e, s, w) for w, wv in enumerate(waves) for (e, s) in wv]
            flat += [(rc.key - layer * E, -1, -1) for rc in recs if rc.slot < 0]  # run on the CPU
            assert list(zip(we.tolist(), wslot.tolist(), wwave.tolist())) == flat
            exp_m = [[rc.key, rc.slot, rc.victim, rc.wave] for rc in recs if not rc.hit and rc.slot >= 0]
            assert misses.tolist() == exp_m
    tr = L.moe_cache_trace(cache)
    ref = np.array([[r.step, r.layer, r.key, r.hit, r.slot, r.victim, r.wave] for r in sim.trace])
    assert np.array_equal(tr, ref)
    h, m = L.moe_cache_stats(cache)
    assert h == int(ref[:, 3].sum()) and m == len(ref) - h
    with pytest.raises(L.MoEError):
        L.moe_cache_set_split(cache, 0, 0)
    with pytest.raises(L.MoEError):
        L.moe_cache_set_split(cache, -1, 2)


def test_cache_errors_and_invalidate(L):
    with pytest.raises(L.MoEError) as ei:
        L.MoeCache(1, 8, 0)
    assert ei.value.code == L.MOE_ECAPACITY
    with pytest.raises(L.MoEError) as ei:
        L.MoeCache(0, 8, 4)
    assert ei.value.code == L.MOE_EINVAL
    c = L.MoeCache(2, 8, 4)
    for bad, why in [([3, 1], "unsorted"), ([2, 2], "duplicate"), ([8], "expert range"), ([-1], "negative")]:
        with pytest.raises(L.MoEError) as ei:
            L.cache_resolve(c, 0, 0, bad)
        assert ei.value.code == L.MOE_EINVAL, why
    with pytest.raises(L.MoEError):
        L.cache_resolve(c, 0, 2, [1])  # layer out of range
    # a failed fill is undone by invalidating the key: its slot is free again
    we, ws, _, misses, _ = L.cache_resolve(c, 0, 1, [0, 3, 5])
    assert ws.tolist() == [0, 1, 2]
    L.moe_cache_invalidate(c, 1 * 8 + 3)
    assert L.moe_cache_slot_of(c, 1 * 8 + 3) == -1
    with pytest.raises(L.MoEError):
        L.moe_cache_invalidate(c, 1 * 8 + 3)  # not resident any more
    _, ws, _, misses, _ = L.cache_resolve(c, 1, 0, [7])
    assert ws.tolist() == [1] and misses.tolist() == [[7, 1, -1, 0]]  # lowest free slot
    L.moe_cache_clear_trace(c)
    assert len(L.moe_cache_trace(c)) == 0


def test_failed_fill_leaves_keys_unmapped(L):
    """cache_fill_async that cannot issue its copies (here: no pool address for the layer; without a GPU the
    event set-up fails first) drops the batch's keys, so none stays resident without its blob."""
    c = L.MoeCache(2, 8, 4)
    _, ws, _, misses, _ = L.cache_resolve(c, 0, 0, [2])
    _, ws, _, misses, _ = L.cache_resolve(c, 0, 1, [0, 3, 5])
    assert ws.tolist() == [1, 2, 3] and len(misses) == 3
    ms = np.ascontiguousarray(np.asarray(misses, np.int32))
    lp = L.layer_table([0x1000, 0])  # layer 1 has no pool address
    rc = L._lib.cache_fill_async(c.h, ms.ctypes.data, len(ms), lp.ctypes.data, 4096, 4096, 0x10000, 4096, None, None)
    assert rc in (L.MOE_EINVAL, L.MOE_EHIP)
    assert [L.moe_cache_slot_of(c, 8 + e) for e in (0, 3, 5)] == [-1, -1, -1]
    assert L.moe_cache_slot_of(c, 2) == 0  # an earlier entry is untouched
    _, ws, _, misses, _ = L.cache_resolve(c, 1, 1, [7])
    assert ws.tolist() == [1] and misses.tolist() == [[15, 1, -1, 0]]  # lowest free slot


def test_argument_validation_without_gpu(L):
    lib = L._lib
    # routing: k > E, bad dtype, workspace too small -- all rejected before any launch
    assert lib.moe_route(None, 1, None, None, 4, 64, 8, 9, None, None, None, 1, 1, None, None, 1, 1 << 20, None) \
        == L.MOE_EINVAL
    assert lib.moe_route(1, 5, 1, None, 4, 64, 8, 2, 1, 1, None, 1, 1, 1, 1, 1, 1 << 20, None) == L.MOE_EINVAL
    assert lib.moe_route(1, 1, 1, None, 4, 64, 8, 2, 1, 1, None, 1, 1, 1, 1, 1, 16, None) == L.MOE_EINVAL
    assert "workspace" in L.moe_last_error()
    # FFN: dtype / format mismatch, bad mode, slot stride smaller than a blob
    w = np.array([[0, 0, 0, 1]], np.int32)
    assert lib.moe_ffn(1, L.MOE_DT_F32, 1, w.ctypes.data, 1, 1, 1 << 30, L.MOE_W_BF16, 256, 128, 1, 1, 1 << 30, 0,
                       None) == L.MOE_EINVAL
    assert lib.moe_ffn(1, L.MOE_DT_BF16, 1, w.ctypes.data, 1, 1, 1 << 30, L.MOE_W_BF16, 256, 128, 1, 1, 1 << 30, 9,
                       None) == L.MOE_EINVAL
    assert lib.moe_ffn(1, L.MOE_DT_BF16, 1, w.ctypes.data, 1, 1, 1024, L.MOE_W_BF16, 256, 128, 1, 1, 1 << 30, 0,
                       None) == L.MOE_EINVAL
    # prefill GEMM on shapes it does not tile (H % 128 != 0) is refused, not attempted
    assert lib.moe_ffn(1, L.MOE_DT_BF16, 1, w.ctypes.data, 1, 1, 1 << 30, L.MOE_W_BF16, 96, 128, 1, 1, 1 << 30,
                       L.MOE_FFN_PREFILL, None) == L.MOE_EINVAL
    # combine: bad output dtype
    assert lib.moe_combine(1, 1, 1, 2, 2, 8, 1, 9, None) == L.MOE_EINVAL
    # fills: slot index beyond the cache
    c = L.MoeCache(1, 8, 2)
    m = np.array([[0, 5, -1, 0]], np.int32)
    assert lib.cache_fill_async(c.h, m.ctypes.data, 1, 1, 64, 64, 1, 64, None, None) == L.MOE_EINVAL
    # pipe and decoder: null arguments
    st = ctypes.c_int(0)
    assert lib.moe_pipe_create(None, 64, 2, ctypes.byref(st)) is None and st.value == L.MOE_EINVAL
    assert lib.moe_decoder_create(None, 1, 64, 64, 8, 2, 1, 1, None, 0, None, 0, None, ctypes.byref(st)) is None
    assert st.value == L.MOE_EINVAL
    assert lib.moe_decoder_step(None, 0, 0, None, 1, None, None, None, 0, None, None) == L.MOE_EINVAL
    assert lib.moe_decoder_profile(None, 8) == L.MOE_EINVAL


@pytest.mark.parametrize("S,sizes,E,Lyr,max_active", [
    (16, [5, 12, 1, 16], 32, 2, 5), (8, [8, 3, 20], 16, 1, 3), (64, [10, 64], 256, 1, 6), (4, [2, 9], 12, 3, 2)])
def test_cache_resize_matches_oracle(L, S, sizes, E, Lyr, max_active):
    """Resizes between layer-steps: moves, capacity and every later access equal the oracle's."""
    r = np.random.default_rng(S * 7 + E)
    cache = L.MoeCache(Lyr, E, S)
    sim = oracle.SharedLRU(S)
    zipf = 1.0 / np.arange(1, E + 1) ** 1.1
    step = 0
    for S_new in [None] + sizes:
        if S_new is not None:
            moves = L.moe_cache_resize(cache, S_new)
            ref = sim.resize(S_new)
            assert moves.tolist() == [list(m) for m in ref]
            assert L.moe_cache_capacity(cache) == S_new
            for key in range(Lyr * E):
                assert L.moe_cache_slot_of(cache, key) == sim.key_slot.get(key, -1)
        for _ in range(15):
            for layer in range(Lyr):
                n = int(r.integers(1, max_active + 1))
                ex = np.sort(r.choice(E, size=n, replace=False, p=zipf / zipf.sum())).astype(np.int32)
                L.cache_resolve(cache, step, layer, ex)
                sim.resolve(step, layer, E, ex)
            step += 1
    tr = L.moe_cache_trace(cache)
    ref = np.array([[q.step, q.layer, q.key, q.hit, q.slot, q.victim, q.wave] for q in sim.trace])
    assert np.array_equal(tr, ref)
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_resize(cache, 0)
    assert ei.value.code == L.MOE_ECAPACITY


def test_device_decoder_and_graph_validation_without_gpu(L):
    """The device-controlled decoder, graph and resize entry points reject bad arguments before any HIP call."""
    lib = L._lib
    st = ctypes.c_int(0)
    bufs = L.DecoderBuffers()  # all-null buffers
    pool = np.array([1, 1], np.uint64)  # two layer addresses (never read: creation fails earlier)
    args = dict(L=2, E=16, S=6, T=3, H=256, I=128, k=2, dt=L.MOE_DT_BF16, wf=L.MOE_W_BF16)

    def create(**kw):
        a = dict(args, **kw)
        return lib.moe_device_decoder_create(a["L"], a["E"], a["S"], a["T"], a["H"], a["I"], a["k"], a["dt"], a["wf"],
                                             pool.ctypes.data, 1 << 20, 1, 1 << 20, ctypes.byref(bufs), 0,
                                             ctypes.byref(st))

    # a layer-step's experts must fit the cache at once: S >= min(E, k*T)
    assert create(S=5) is None and st.value == L.MOE_ECAPACITY
    assert "min(E, k*T_max)" in L.moe_last_error()
    assert create(S=0) is None and st.value == L.MOE_ECAPACITY
    assert create(E=2000) is None and st.value == L.MOE_EINVAL          # resolve kernel: one thread per expert
    assert create(k=17) is None and st.value == L.MOE_EINVAL
    assert create(dt=L.MOE_DT_F32) is None and st.value == L.MOE_EINVAL  # fp32 activations need fp32 weights
    assert create(wf=9) is None and st.value == L.MOE_EINVAL
    assert create() is None and st.value == L.MOE_EINVAL                 # null device buffers
    assert lib.moe_device_decoder_create(2, 16, 6, 3, 256, 128, 2, 1, 1, None, 1 << 20, 1, 1 << 20,
                                         ctypes.byref(bufs), 0, ctypes.byref(st)) is None
    assert st.value == L.MOE_EINVAL
    # calls on a null decoder or with null arguments
    assert lib.moe_device_decoder_step(None, 0, 1, 1, 1, 1, 1, 0, None) == L.MOE_EINVAL
    assert lib.moe_device_decoder_resize(None, 8, None, None) == L.MOE_EINVAL
    h, m, r = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    assert lib.moe_device_decoder_stats(None, ctypes.byref(h), ctypes.byref(m), ctypes.byref(r)) == L.MOE_EINVAL
    assert lib.moe_device_decoder_trace(None, None, 0, ctypes.byref(h)) == L.MOE_EINVAL
    assert lib.moe_device_decoder_slot_of(None, 0, ctypes.byref(st)) == L.MOE_EINVAL
    assert lib.moe_device_decoder_destroy(None) == L.MOE_OK
    # graphs: capture needs a created stream; null graphs are refused, destroying NULL is a no-op
    assert lib.moe_graph_begin(None) == L.MOE_EINVAL
    assert lib.moe_graph_end(None, ctypes.byref(st)) is None and st.value == L.MOE_EINVAL
    assert lib.moe_graph_launch(None, None) == L.MOE_EINVAL
    assert lib.moe_graph_destroy(None) == L.MOE_OK
    # resize of the host policy: null handle and a move array that is too short leave the cache unchanged
    assert lib.moe_cache_resize(None, 4, None, 0, ctypes.byref(st)) == L.MOE_EINVAL
    assert lib.moe_decoder_resize(None, 4, None, None) == L.MOE_EINVAL
    c = L.MoeCache(1, 8, 4)
    L.cache_resolve(c, 0, 0, np.array([0, 1, 2, 3], np.int32))
    L.cache_resolve(c, 1, 0, np.array([2], np.int32))  # 2 becomes the most recent
    moves = np.zeros((4, 3), np.int32)
    assert lib.moe_cache_resize(c.h, 2, moves.ctypes.data, 0, ctypes.byref(st)) == L.MOE_EINVAL
    assert L.moe_cache_capacity(c) == 4 and L.moe_cache_slot_of(c, 3) == 3
    mv = L.moe_cache_resize(c, 2)  # keeps 2 (slot 2) and 3 (slot 3): both move below the new size
    assert L.moe_cache_capacity(c) == 2
    assert mv.tolist() == [[2, 2, 0], [3, 3, 1]]
    assert [L.moe_cache_slot_of(c, k) for k in range(4)] == [-1, -1, 0, 1]


def test_binding_refuses_host_and_strided_tensors(L):
    """Device arguments must be GPU tensors and every tensor contiguous: the binding raises before the
    library sees an address that a kernel would misread."""
    import torch
    y = torch.zeros((6, 8), dtype=torch.float32)
    pos = torch.zeros((1, 6), dtype=torch.int32)
    w = torch.zeros((1, 6), dtype=torch.float32)
    out = torch.zeros((1, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        L.moe_combine(y, pos, w, out)
    with pytest.raises(ValueError, match="GPU tensor"):
        L._dptr(np.zeros(4, np.float32))
    with pytest.raises(ValueError, match="contiguous"):
        L._ptr(torch.zeros((4, 4)).t())
    with pytest.raises(ValueError, match="contiguous"):
        L._ptr(np.zeros((4, 4), np.float32).T)
    assert L._dptr(None) is None and L._dptr(1 << 20) == 1 << 20
    assert L._ptr(y) == y.data_ptr()


def test_grouped_ffn_and_prefill_layer_validation_without_gpu(L):
    """moe_ffn_grouped and moe_prefill_layer refuse unsupported formats, shapes, sizes and null arguments
    before any launch."""
    lib = L._lib
    ws = L.moe_ffn_workspace_size(4096 * 6, 4096, 2048, L.MOE_W_BF16)
    assert ws > 0

    def grouped(**kw):
        a = dict(x=1, dt=L.MOE_DT_BF16, ps=1, c=1, o=1, so=None, E=256, ns=256, rows=4096 * 6, base=1,
                 stride=1 << 26, wf=L.MOE_W_BF16, H=4096, I=2048, y=1, w=1, wsb=ws)
        a.update(kw)
        return lib.moe_ffn_grouped(a["x"], a["dt"], a["ps"], a["c"], a["o"], a["so"], a["E"], a["ns"], a["rows"],
                                   a["base"], a["stride"], a["wf"], a["H"], a["I"], a["y"], a["w"], a["wsb"], None)

    assert grouped(wf=L.MOE_W_INT4) == L.MOE_EINVAL          # no GEMM for int4 experts
    assert grouped(wf=L.MOE_W_F32, dt=L.MOE_DT_F32) == L.MOE_EINVAL
    assert grouped(H=4096 + 128) == L.MOE_EINVAL             # H not a multiple of 256
    assert grouped(dt=L.MOE_DT_F32) == L.MOE_EINVAL          # bf16 activations only
    assert grouped(E=0) == L.MOE_EINVAL and grouped(E=1025) == L.MOE_EINVAL
    assert grouped(ns=0) == L.MOE_EINVAL and grouped(rows=-1) == L.MOE_EINVAL
    assert grouped(c=None) == L.MOE_EINVAL and grouped(o=None) == L.MOE_EINVAL and grouped(x=None) == L.MOE_EINVAL
    assert grouped(stride=1024) == L.MOE_EINVAL              # slot stride below one blob
    assert grouped(wsb=ws - 1) == L.MOE_EINVAL
    assert "workspace" in L.moe_last_error()
    assert grouped(rows=0) == L.MOE_OK                       # nothing to compute, nothing launched
    bufs = L.DecoderBuffers()
    assert lib.moe_prefill_layer(1, L.MOE_DT_BF16, 1, None, 16, 4096, 256, 6, 2048, L.MOE_W_BF16, 1, 1 << 26,
                                 None, 1, L.MOE_DT_F32, None) == L.MOE_EINVAL   # null buffer struct
    assert lib.moe_prefill_layer(1, L.MOE_DT_BF16, 1, None, 16, 4096, 256, 6, 2048, L.MOE_W_INT4, 1, 1 << 26,
                                 ctypes.byref(bufs), 1, L.MOE_DT_F32, None) == L.MOE_EINVAL
    assert lib.moe_prefill_layer(1, L.MOE_DT_BF16, 1, None, 16, 4096, 256, 6, 2048, L.MOE_W_BF16, 1, 1 << 26,
                                 ctypes.byref(bufs), 1, L.MOE_DT_F32, None) == L.MOE_EINVAL   # null y_perm
    assert lib.moe_prefill_layer(1, L.MOE_DT_BF16, 1, None, -1, 4096, 256, 6, 2048, L.MOE_W_BF16, 1, 1 << 26,
                                 ctypes.byref(bufs), 1, L.MOE_DT_F32, None) == L.MOE_EINVAL
