"""GPU parity of the device-controlled decode step (cache tables, resolve and
fills on the GPU, no host synchronisation inside a step) and of its
graph-captured replay.

The device-resident LRU must produce the oracle's trace bit for bit, the
layer outputs must match the oracle, and graph replays must equal eager steps
of an identical decoder bit for bit (same kernels, same inputs, same cache
state), with eager work and synchronisation between the replays.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.parity import check_close, check_permutation, check_routing, np64, npi
from tests.test_gpu_layer import ExpertCache64, make_store, oracle_out_rows
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu
dev = "cuda"


def small_bf16(S):
    return dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name=f"devsmall_s{S}", L=3, T=3, steps=40, H=256,
                               E=16, I=128, k=2, zipf_s=1.2, epoch=8, S=S)


def small_int4():
    return dataclasses.replace(CONFIGS["decode_int4_t8_l8"], name="devsmall_int4", L=2, T=4, steps=24, H=256, E=16,
                               I=256, k=4, zipf_s=1.0, epoch=6, S=16, weights_of=None, pool_layers=None)


def small_mxfp4():
    return dataclasses.replace(CONFIGS["decode_mxfp4_t8_l8"], name="devsmall_mxfp4", L=2, T=4, steps=24, H=256,
                               E=16, I=256, k=4, zipf_s=1.0, epoch=6, S=16, weights_of=None, pool_layers=None)


def oracle_trace(sim):
    return np.array([[r.step, r.layer, r.key, r.hit, r.slot, r.victim, r.wave] for r in sim.trace], np.int64)


def device_trace(dl, L, cap):
    t, n = dl.trace(cap)
    assert n <= cap, f"trace capacity {cap} too small for {n} accesses"
    t = t.astype(np.int64)
    seq = t[:, 0].copy()
    assert np.array_equal(t[:, 1], seq % L), "resolve calls out of layer order"
    t[:, 0] = seq // L
    return t


def run_device(cfg, steps, out_check, check_all=False, trace_cap=1 << 16, resizes=None):
    """Eager device-controlled steps over all layers; routing, trace and outputs against the oracle."""
    from routed_expert_layer_amd.runtime import DeviceDecodeLayer
    print(f"device decode {cfg.name}: L={cfg.L} T={cfg.T} steps={steps} S={cfg.S} {cfg.wfmt}", flush=True)
    store = make_store(cfg)
    try:
        dl = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev, trace_capacity=trace_cap)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        Wr64 = [np64(w) for w in Wr]
        sim = oracle.SharedLRU(cfg.S)
        experts64 = {}
        for step in range(steps):
            if steps >= 128 and (step + 1) % 128 == 0:
                print(f"  step {step + 1}/{steps}", flush=True)
            if resizes and step in resizes:
                dl.resize(resizes[step])
                sim.resize(resizes[step])
            for layer in range(cfg.L):
                b = gen.router_bias(cfg, layer, step, dev)
                x = gen.tokens(cfg, step, layer, dev)
                out = dl.step(layer, x, Wr[layer], b)
                torch.cuda.synchronize()
                l64 = oracle.router_logits(x, Wr64[layer], b)
                idx = npi(dl.rb.topk_idx[:cfg.T])
                check_routing(idx, np64(dl.rb.topk_w[:cfg.T]), l64, cfg.k)
                counts, _, _, _ = check_permutation(idx, npi(dl.rb.counts), npi(dl.rb.offsets),
                                                    npi(dl.rb.perm_src[:cfg.T * cfg.k]), npi(dl.rb.perm_pos[:cfg.T]),
                                                    cfg.E)
                sim.resolve(step, layer, cfg.E, np.nonzero(counts)[0])
                if check_all or (step, layer) in out_check:
                    ge = experts64.setdefault(layer, ExpertCache64(cfg, layer))
                    ref = oracle_out_rows(np64(x), idx, l64, list(range(cfg.T)), ge)
                    check_close(np64(out), ref, f"{cfg.name} step {step} layer {layer}")
        ref = oracle_trace(sim)
        got = device_trace(dl, cfg.L, trace_cap)
        assert got.shape == ref.shape, f"trace length {got.shape} vs {ref.shape}"
        assert np.array_equal(got, ref), "device cache trace differs from the oracle's LRU"
        hits, misses, calls = dl.stats()
        assert hits == int(ref[:, 3].sum()) and misses == len(ref) - hits and calls == steps * cfg.L
        print(f"  trace ok: {len(ref)} accesses, hit rate {hits / max(len(ref), 1):.3f}, fills {misses}", flush=True)
        return ref
    finally:
        store.close()


@pytest.mark.parametrize("S", [6, 8], ids=["S_eq_kT", "S8"])
def test_device_small_bf16_all_outputs(S):
    ref = run_device(small_bf16(S), 40, set(), check_all=True)
    assert (ref[:, 5] >= 0).any(), "the small config should evict"


@pytest.mark.parametrize("fused", [False, True], ids=["combine", "fused"])
def test_device_resize_all_outputs(fused):
    """Shrink to the smallest allowed size (k*T), then grow into a new buffer, between steps."""
    if fused:  # one-token steps whose down projection forms the output (k*T = 4)
        ref = run_device(dataclasses.replace(fused_bf16(1024), S=8), 36, set(), check_all=True,
                         resizes={12: 4, 24: 10})
    else:
        ref = run_device(small_bf16(10), 36, set(), check_all=True, resizes={12: 6, 24: 14})
    assert (ref[:, 5] >= 0).any()


def test_device_small_int4_all_outputs():
    ref = run_device(small_int4(), 24, set(), check_all=True)
    assert (ref[:, 5] >= 0).any(), "the small int4 config should evict"


def test_device_small_mxfp4_all_outputs():
    ref = run_device(small_mxfp4(), 24, set(), check_all=True)
    assert (ref[:, 5] >= 0).any(), "the small MXFP4 config should evict"


@pytest.mark.timeout(600)
def test_device_decode_bf16_full():
    cfg = CONFIGS["decode_bf16_h4096_e256"]
    run_device(cfg, cfg.steps, {(s, 0) for s in (0, 1, 2, 63, 200, 383, 1023)})


@pytest.mark.timeout(900)
def test_device_decode_int4_full():
    cfg = CONFIGS["decode_int4_t8_l8"]
    run_device(cfg, cfg.steps, {(0, 2), (130, 2), (255, 2)})


def fused_bf16(I):
    """Single-token bf16 steps whose down projection forms the output (misses written through on the way)."""
    return dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name=f"devfused_i{I}", L=2, T=1, steps=40, H=256,
                               E=16, I=I, k=4, zipf_s=1.0, epoch=8, S=6)


@pytest.mark.parametrize("I", [512, 2048])
def test_device_fused_combine_all_outputs(I):
    """The device step's down projection writes the output, hits and written-through misses alike: every
    output and the whole trace against the oracle (later hits read the slots the misses were written into)."""
    cfg = fused_bf16(I)
    ref = run_device(cfg, cfg.steps, set(), check_all=True)
    assert (ref[:, 3] == 0).sum() > 10 and (ref[:, 3] == 1).sum() > 40


def test_device_fused_combine_bf16_output():
    """Two identical device decoders over one pool, one writing fp32 outputs and one bf16: the bf16 output is
    the fp32 one rounded to nearest even, with the output formed in the down projection."""
    from routed_expert_layer_amd.runtime import DeviceDecodeLayer
    cfg = fused_bf16(2048)
    store = make_store(cfg)
    try:
        A = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
        B = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        oa = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
        ob = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
        for step in range(30):
            for layer in range(cfg.L):
                b = gen.router_bias(cfg, layer, step, dev)
                x = gen.tokens(cfg, step, layer, dev)
                A.step(layer, x, Wr[layer], b, out=oa)
                B.step(layer, x, Wr[layer], b, out=ob)
                torch.cuda.synchronize()
                assert torch.equal(ob, oa.to(torch.bfloat16)), f"step {step} layer {layer}"
        ha, ma, _ = A.stats()
        assert ma > 0 and (ha, ma) == B.stats()[:2]
    finally:
        store.close()


@pytest.mark.parametrize("fused", ["combine", "fused", "int4"])
def test_graph_replay_equals_eager(fused):
    """Two identical device decoders over one pool: A steps eagerly, B replays one captured graph holding all
    layers; outputs and traces must agree bit for bit on every step, and both with the oracle's trace (with
    the separate combine, with the output formed in the down projection, and with int4 experts, whose two
    projections run as one launch numbered by the resolve's device-side call counter)."""
    from routed_expert_layer_amd.runtime import DeviceDecodeLayer
    cfg = {"combine": small_bf16(6), "fused": fused_bf16(1024), "int4": small_int4()}[fused]
    steps = 24
    store = make_store(cfg)
    try:
        A = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev, trace_capacity=4096)
        B = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev, trace_capacity=4096)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        xs = [torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev) for _ in range(cfg.L)]
        bs = [torch.empty(cfg.E, dtype=torch.float32, device=dev) for _ in range(cfg.L)]
        outs = [torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
        cs = torch.cuda.Stream()
        torch.cuda.synchronize()

        def enqueue():
            for l in range(cfg.L):
                B.step(l, xs[l], Wr[l], bs[l], cs, out=outs[l])

        graph = DeviceDecodeLayer.capture(enqueue, cs)
        sim = oracle.SharedLRU(cfg.S)
        for step in range(steps):
            for l in range(cfg.L):
                xs[l].copy_(gen.tokens(cfg, step, l, dev))
                bs[l].copy_(gen.router_bias(cfg, l, step, dev))
            torch.cuda.synchronize()
            DeviceDecodeLayer.replay(graph, cs)
            cs.synchronize()
            got = [o.clone() for o in outs]
            for l in range(cfg.L):
                oa = A.step(l, xs[l], Wr[l], bs[l]).clone()
                torch.cuda.synchronize()
                counts = npi(A.rb.counts)
                sim.resolve(step, l, cfg.E, np.nonzero(counts)[0])
                assert torch.equal(oa, got[l]), f"graph replay differs from the eager step at step {step} layer {l}"
        ref = oracle_trace(sim)
        ta, tb = device_trace(A, cfg.L, 4096), device_trace(B, cfg.L, 4096)
        assert np.array_equal(ta, ref) and np.array_equal(tb, ref), "traces differ from the oracle's"
        assert A.stats() == B.stats()
        print(f"  {steps} replays equal the eager steps; {len(ref)} accesses, fills {A.stats()[1]}", flush=True)
        graph.close()
    finally:
        store.close()


@pytest.mark.timeout(900)
def test_stack48_device_graph():
    """48-layer stack through one captured 48-layer graph, across the bias re-draw at step 128: trace against
    the oracle and sampled outputs (some right after the re-draw)."""
    from routed_expert_layer_amd.runtime import DeviceDecodeLayer
    cfg = CONFIGS["stack48_bf16_h2048_e128"]
    steps = 136
    r = np.random.default_rng(5)
    sample = {(int(s), int(l)) for s, l in zip(r.integers(0, steps, 5), r.integers(0, cfg.L, 5))}
    sample |= {(128, 0), (129, 47)}
    print(f"stack48 graph: {steps} steps, output samples {sorted(sample)}", flush=True)
    store = make_store(cfg)
    try:
        dl = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev, trace_capacity=1 << 18)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        xs = [torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev) for _ in range(cfg.L)]
        bs = [torch.empty(cfg.E, dtype=torch.float32, device=dev) for _ in range(cfg.L)]
        outs = [torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
        topk = [torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev) for _ in range(cfg.L)]
        topw = [torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
        cs = torch.cuda.Stream()
        torch.cuda.synchronize()

        def enqueue():
            for l in range(cfg.L):
                dl.step(l, xs[l], Wr[l], bs[l], cs, out=outs[l])
                topk[l].copy_(dl.rb.topk_idx)  # captured with the step: the selection of layer l survives
                topw[l].copy_(dl.rb.topk_w)

        with torch.cuda.stream(cs):
            graph = DeviceDecodeLayer.capture(enqueue, cs)
        sim = oracle.SharedLRU(cfg.S)
        experts64 = {}
        Wr64 = [np64(w) for w in Wr]
        for step in range(steps):
            for l in range(cfg.L):
                xs[l].copy_(gen.tokens(cfg, step, l, dev))
                bs[l].copy_(gen.router_bias(cfg, l, step, dev))
            torch.cuda.synchronize()
            DeviceDecodeLayer.replay(graph, cs)
            cs.synchronize()
            if (step + 1) % 32 == 0:
                print(f"  step {step + 1}/{steps}", flush=True)
            for l in range(cfg.L):
                idx = npi(topk[l])
                l64 = oracle.router_logits(xs[l], Wr64[l], bs[l])
                check_routing(idx, np64(topw[l]), l64, cfg.k)
                sim.resolve(step, l, cfg.E, np.unique(idx))
                if (step, l) in sample:
                    ge = experts64.setdefault(l, ExpertCache64(cfg, l, cap=40))
                    ref = oracle_out_rows(np64(xs[l]), idx, l64, list(range(cfg.T)), ge)
                    check_close(np64(outs[l]), ref, f"stack48 graph step {step} layer {l}")
        ref = oracle_trace(sim)
        got = device_trace(dl, cfg.L, 1 << 18)
        assert np.array_equal(got, ref), "device cache trace differs from the oracle's LRU"
        print(f"  trace ok: {len(ref)} accesses, fills {dl.stats()[1]}", flush=True)
        graph.close()
    finally:
        store.close()


def test_device_decoder_rejects():
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import DeviceDecodeLayer
    cfg = small_bf16(6)
    store = make_store(cfg)
    try:
        with pytest.raises(L.MoEError, match="min"):
            DeviceDecodeLayer(store, 5, cfg.T, cfg.k, cfg.act, dev)  # k*T = 6 > 5 slots
        dl = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
        Wr = gen.router_weight(cfg, 0, dev)
        b = gen.router_bias(cfg, 0, 0, dev)
        with pytest.raises(L.MoEError, match="outside"):
            dl.step(0, gen.tokens(cfg, 0, 0, dev, T=cfg.T + 1), Wr, b)
        with pytest.raises(L.MoEError, match="layer"):
            dl.step(cfg.L, gen.tokens(cfg, 0, 0, dev), Wr, b)
        torch.cuda.synchronize()
        assert dl.stats() == (0, 0, 0)
    finally:
        store.close()
