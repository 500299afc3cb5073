"""End-to-end GPU parity of the layer on the workload configurations.

Routing, permutation and the cache trace are compared on every step; the
layer output is compared on every step for the tiny config and on seeded
samples of steps / tokens at full size, where the oracle evaluates only the
experts the sampled tokens use.
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


class ExpertCache64:
    """fp64 canonical weights of experts, regenerated on demand (bounded)."""

    def __init__(self, cfg, layer, cap=48):
        self.cfg, self.layer, self.cap, self.d = cfg, layer, cap, {}

    def __call__(self, e):
        e = int(e)
        if e not in self.d:
            if len(self.d) >= self.cap:
                self.d.pop(next(iter(self.d)))
            if self.cfg.wfmt == "int4":
                w = gen.expert_int4(self.cfg, self.layer, e, dev)
                g = self.cfg.group
                self.d[e] = (oracle.dequant_int4(w["q1"], w["s1"], g), oracle.dequant_int4(w["q3"], w["s3"], g),
                             oracle.dequant_int4(w["q2"], w["s2"], g))
            elif self.cfg.wfmt == "mxfp4":
                w = gen.expert_mxfp4(self.cfg, self.layer, e, dev)
                self.d[e] = (oracle.dequant_mxfp4(w["c1"], w["s1"]), oracle.dequant_mxfp4(w["c3"], w["s3"]),
                             oracle.dequant_mxfp4(w["c2"], w["s2"]))
            else:
                self.d[e] = tuple(np64(t) for t in gen.expert_weights(self.cfg, self.layer, e, dev))
        return self.d[e]


def oracle_out_rows(x64, idx, l64, tokens, get_expert):
    """Oracle outputs of the listed tokens for the given selection (fp64 weights of that selection)."""
    w = oracle.topk_weights(l64[tokens], idx[tokens])
    out = np.zeros((len(tokens), x64.shape[1]))
    for n, t in enumerate(tokens):
        for j, e in enumerate(idx[t]):
            out[n] += w[n, j] * oracle.swiglu_expert(x64[t:t + 1], *get_expert(e))[0]
    return out


def make_store(cfg):
    """Pinned pool of the config; layers sharing weight sets share pool memory."""
    from routed_expert_layer_amd.runtime import ExpertStore
    store = ExpertStore(cfg.L, cfg.E, cfg.H, cfg.I, cfg.wfmt, phys_layers=cfg.pool_layers)
    for layer in range(store.P):
        print(f"  packing layer {layer} ({cfg.E} experts)", flush=True)
        if cfg.wfmt == "int4":
            store.pack_layer(layer, lambda e: gen.expert_int4(cfg, layer, e, dev))
        elif cfg.wfmt == "mxfp4":
            store.pack_layer(layer, lambda e: gen.expert_mxfp4(cfg, layer, e, dev))
        else:
            store.pack_layer(layer, lambda e: gen.expert_weights(cfg, layer, e, dev))
    return store


def run_decode(cfg, steps, out_check, check_all_outputs=False, native=True, split=None, cpu_check=(0, ()),
               resizes=None):
    """Drive DecodeLayer over `steps` x all layers; check routing, trace, and sampled outputs.

    native=True runs each layer-step through the library's decode driver
    (moe_decoder_step); native=False sequences the individual C-ABI calls from
    Python. split=(rate_gpu, rate_cpu) divides misses between GPU fills and CPU
    execution; cpu_check=(n, layers) also checks the outputs of the first n
    layer-steps of those layers in which some miss ran on the CPU."""
    from routed_expert_layer_amd.runtime import DecodeLayer
    print(f"decode {cfg.name}: L={cfg.L} T={cfg.T} steps={steps} S={cfg.S} {cfg.wfmt} native={native} "
          f"split={split}", flush=True)
    store = make_store(cfg)
    try:
        dl = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev, keep_logits=True, native=native)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        sim = oracle.SharedLRU(cfg.S)
        if split:
            dl.set_split(*split)
            sim.set_split(*split)
        cpu_left, cpu_layers = cpu_check
        experts64 = {}
        for step in range(steps):
            if resizes and step in resizes:
                dl.resize(resizes[step])
                sim.resize(resizes[step])
            for layer in range(cfg.L):
                b = gen.router_bias(cfg, layer, step, dev)
                x = gen.tokens(cfg, step, layer, dev)
                out = dl.step(step, layer, x, Wr[layer], b)
                torch.cuda.synchronize()
                l64 = oracle.router_logits(x, Wr[layer], b)
                idx = npi(dl.rb.topk_idx[:cfg.T])
                check_routing(idx, np64(dl.rb.topk_w[:cfg.T]), l64, cfg.k)
                counts, _, _, _ = check_permutation(idx, npi(dl.rb.counts), npi(dl.rb.offsets),
                                                    npi(dl.rb.perm_src[:cfg.T * cfg.k]), npi(dl.rb.perm_pos[:cfg.T]),
                                                    cfg.E)
                _, recs = sim.resolve(step, layer, cfg.E, np.nonzero(counts)[0])
                on_cpu = any(rc.slot < 0 for rc in recs)
                check_cpu = on_cpu and cpu_left > 0 and layer in cpu_layers
                cpu_left -= int(check_cpu)
                if check_all_outputs or (step, layer) in out_check or check_cpu:
                    ge = experts64.setdefault(layer, ExpertCache64(cfg, layer))
                    ref = oracle_out_rows(np64(x), idx, l64, list(range(cfg.T)), ge)
                    check_close(np64(out), ref, f"{cfg.name} step {step} layer {layer}")
        trace = dl.trace()
        ref = np.array([[r.step, r.layer, r.key, r.hit, r.slot, r.victim, r.wave] for r in sim.trace], np.int64)
        assert trace.shape == ref.shape, f"trace length {trace.shape} vs {ref.shape}"
        assert np.array_equal(trace, ref), "cache trace differs from the oracle's LRU"
        hits = int(ref[:, 3].sum())
        cpu = int((ref[:, 4] < 0).sum())
        print(f"  trace ok: {len(ref)} accesses, hit rate {hits / max(len(ref), 1):.3f}, fills {dl.n_fills}, "
              f"cpu runs {dl.cpu_runs}, waves>1 in {int((ref[:, 6] > 0).sum())} accesses", flush=True)
        assert dl.n_fills == len(ref) - hits - cpu
        assert dl.cpu_runs == cpu
        assert cpu_left <= 0 or not cpu_layers, "no CPU-run layer-step was output-checked"
        return ref
    finally:
        store.close()


@pytest.mark.parametrize("native", [True, False], ids=["driver", "python"])
def test_tiny_fp32_all_steps(native):
    cfg = CONFIGS["tiny_f32_h256_e16"]
    ref = run_decode(cfg, cfg.steps, set(), check_all_outputs=True, native=native)
    assert (ref[:, 6] > 0).any(), "the tiny config should exercise multi-wave layer-steps"


@pytest.mark.timeout(600)
def test_decode_bf16_full():
    cfg = CONFIGS["decode_bf16_h4096_e256"]
    run_decode(cfg, cfg.steps, {(s, 0) for s in (0, 1, 2, 63, 511, 1023)})


@pytest.mark.timeout(600)
def test_stack48_bf16_cut():
    cfg = CONFIGS["stack48_bf16_h2048_e128"]
    r = np.random.default_rng(3)
    sample = {(int(s), int(l)) for s, l in zip(r.integers(0, 40, 6), r.integers(0, 48, 6))}
    run_decode(cfg, 40, sample)


@pytest.mark.timeout(600)
def test_decode_int4_cut():
    cfg = CONFIGS["decode_int4_t8_l8"]
    run_decode(cfg, 48, {(0, 0), (5, 3), (47, 7)})


@pytest.mark.timeout(600)
def test_decode_mxfp4_cut():
    cfg = CONFIGS["decode_mxfp4_t8_l8"]
    run_decode(cfg, 48, {(0, 0), (5, 3), (47, 7)})


@pytest.mark.parametrize("native", [True, False], ids=["driver", "python"])
def test_resize_small_all_outputs(native):
    """The cache shrinks (entries above the new size move), then grows into a new buffer; every output and
    the whole trace against the oracle."""
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name="resize_small", L=3, T=3, H=256, I=128, E=16,
                              k=2, zipf_s=1.2, epoch=8, S=10)
    run_decode(cfg, 36, set(), check_all_outputs=True, native=native, resizes={12: 4, 24: 14})


@pytest.mark.timeout(600)
def test_split_small_all_outputs():
    """Misses divided 1:3 between GPU fills and CPU execution; every output checked."""
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name="split_small", L=3, T=4, H=512, I=256, E=32,
                              k=4, zipf_s=1.0, S=8)
    ref = run_decode(cfg, 24, set(), check_all_outputs=True, split=(1, 3))
    assert (ref[:, 4] < 0).sum() > 10 and (ref[:, 3] == 0).sum() > (ref[:, 4] < 0).sum()


@pytest.mark.timeout(600)
def test_stack48_split_cut():
    """The 48-layer stack with misses divided in the ratio of a measured fill and CPU rate (56 : 165 GB/s)."""
    cfg = CONFIGS["stack48_bf16_h2048_e128"]
    run_decode(cfg, 10, {(9, 47)}, split=(56, 165), cpu_check=(4, (0, 1, 2)))


def _prefill_check(cfg, layer, pl, x, Wr, b, n_sample=24):
    T = cfg.T
    l64 = oracle.router_logits(x, Wr, b)
    idx = npi(pl.rb.topk_idx[:T])
    check_routing(idx, np64(pl.rb.topk_w[:T]), l64, cfg.k)
    check_permutation(idx, npi(pl.rb.counts), npi(pl.rb.offsets), npi(pl.rb.perm_src[:T * cfg.k]),
                      npi(pl.rb.perm_pos[:T]), cfg.E)
    r = np.random.default_rng(1000 + layer)
    tokens = sorted(r.choice(T, n_sample, replace=False).tolist())
    # include tokens of the smallest and largest groups
    counts = npi(pl.rb.counts)
    for e in (int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))):
        tokens.append(int(np.nonzero((idx == e).any(1))[0][0]))
    tokens = sorted(set(tokens))
    ref = oracle_out_rows(np64(x), idx, l64, tokens, ExpertCache64(cfg, layer, cap=64))
    check_close(np64(pl.out[tokens]), ref, f"{cfg.name} layer {layer}")
    return counts


@pytest.mark.timeout(600)
def test_prefill_4096_resident():
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import PrefillLayer
    cfg = CONFIGS["prefill_bf16_t4096_e256"]
    blob = L.moe_expert_bytes(L.MOE_W_BF16, cfg.H, cfg.I)
    stride = (blob + 4095) // 4096 * 4096
    buf = torch.empty(cfg.E * stride, dtype=torch.uint8, device=dev)
    for e in range(cfg.E):
        W1, W3, W2 = gen.expert_weights(cfg, 0, e, dev)
        L.moe_pack_expert(L.MOE_W_BF16, cfg.H, cfg.I, W1, W3, W2, None, None, None, buf[e * stride:])
    pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, stride, dev, keep_logits=True)
    Wr = gen.router_weight(cfg, 0, dev)
    b = gen.router_bias(cfg, 0, 0, dev)
    x = gen.tokens(cfg, 0, 0, dev)
    pl.forward(x, Wr, b, buf)
    torch.cuda.synchronize()
    counts = _prefill_check(cfg, 0, pl, x, Wr, b)
    print(f"  tokens per expert: min {counts.min()} max {counts.max()} mean {counts.mean():.1f}", flush=True)


@pytest.mark.timeout(600)
def test_prefill_4096_mxfp4_resident():
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import PrefillLayer
    cfg = CONFIGS["prefill_mxfp4_t4096_e256"]
    blob = L.moe_expert_bytes(L.MOE_W_MXFP4, cfg.H, cfg.I)
    stride = (blob + 4095) // 4096 * 4096
    buf = torch.empty(cfg.E * stride, dtype=torch.uint8, device=dev)
    for e in range(cfg.E):
        w = gen.expert_mxfp4(cfg, 0, e, dev)
        L.moe_pack_expert(L.MOE_W_MXFP4, cfg.H, cfg.I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"],
                          buf[e * stride:])
    pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, stride, dev, keep_logits=True, wfmt=L.MOE_W_MXFP4)
    Wr = gen.router_weight(cfg, 0, dev)
    b = gen.router_bias(cfg, 0, 0, dev)
    x = gen.tokens(cfg, 0, 0, dev)
    pl.forward(x, Wr, b, buf, wfmt=L.MOE_W_MXFP4)
    torch.cuda.synchronize()
    counts = _prefill_check(cfg, 0, pl, x, Wr, b)
    print(f"  tokens per expert: min {counts.min()} max {counts.max()} mean {counts.mean():.1f}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_db_bf16_t16384_l8", "prefill_db_mxfp4_t16384_l8"])
def test_prefill_16384_double_buffered(name):
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import PrefillLayer
    cfg = CONFIGS[name]
    store = make_store(cfg)
    try:
        pipe = L.MoePipe(store.layer_ptrs, store.layer_bytes)
        pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, store.stride, dev, keep_logits=True, wfmt=store.wfmt)
        s = torch.cuda.current_stream()
        for layer in range(cfg.L):
            Wr = gen.router_weight(cfg, layer, dev)
            b = gen.router_bias(cfg, layer, 0, dev)
            x = gen.tokens(cfg, 0, layer, dev)
            base = L.moe_pipe_begin_layer(pipe, layer, s)
            pl.forward(x, Wr, b, base, wfmt=store.wfmt)
            L.moe_pipe_end_layer(pipe, layer, s)
            torch.cuda.synchronize()
            counts = _prefill_check(cfg, layer, pl, x, Wr, b, n_sample=8)
            print(f"  layer {layer}: active experts {int((counts > 0).sum())}, max group {counts.max()}, "
                  f"copy {L.moe_pipe_copy_ms(pipe, layer):.1f} ms", flush=True)
        pipe.close()
    finally:
        store.close()
