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
               resizes=None, invalidate=None):
    """Drive a decode layer over `steps` x all layers; check routing, trace, and sampled outputs.

    native=True runs each layer-step through the library's decode driver
    (moe_decoder_step); native=False sequences the individual C-ABI calls from
    Python (tests/sequenced.py). split=(rate_gpu, rate_cpu) divides misses
    between GPU fills and CPU execution; cpu_check=(n, layers) also checks the
    outputs of the first n layer-steps of those layers in which some miss ran
    on the CPU. invalidate={step: n} unmaps the n lowest resident keys
    before that step, in the library and in the oracle."""
    from routed_expert_layer_amd.runtime import DecodeLayer
    from tests.sequenced import SequencedDecodeLayer
    print(f"decode {cfg.name}: L={cfg.L} T={cfg.T} steps={steps} S={cfg.S} {cfg.wfmt} native={native} "
          f"split={split} output checks={len(out_check) if not check_all_outputs else 'all'}", flush=True)
    store = make_store(cfg)
    try:
        cls = DecodeLayer if native else SequencedDecodeLayer
        dl = cls(store, cfg.S, cfg.T, cfg.k, cfg.act, dev, keep_logits=True)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        Wr64 = [np64(w) for w in Wr]
        sim = oracle.SharedLRU(cfg.S)
        if split:
            dl.set_split(*split)
            sim.set_split(*split)
        cpu_left, cpu_layers = cpu_check
        experts64 = {}
        n_checked = 0
        for step in range(steps):
            if resizes and step in resizes:
                dl.resize(resizes[step])
                sim.resize(resizes[step])
            if invalidate and step in invalidate:
                from routed_expert_layer_amd import _lib as L
                for key in sorted(sim.key_slot)[:invalidate[step]]:
                    L.moe_cache_invalidate(dl.cache, key)
                    assert sim.drop(key)
            for layer in range(cfg.L):
                b = gen.router_bias(cfg, layer, step, dev)
                x = gen.tokens(cfg, step, layer, dev)
                out = dl.step(step, layer, x, Wr[layer], b)
                torch.cuda.synchronize()
                l64 = oracle.router_logits(x, Wr64[layer], b)
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
                    n_checked += 1
            if steps >= 64 and (step + 1) % 64 == 0:
                print(f"  step {step + 1}/{steps}: routing and grouping match, {n_checked} outputs checked",
                      flush=True)
        trace = dl.trace()
        ref = np.array([[r.step, r.layer, r.key, r.hit, r.slot, r.victim, r.wave] for r in sim.trace], np.int64)
        assert trace.shape == ref.shape, f"trace length {trace.shape} vs {ref.shape}"
        assert np.array_equal(trace, ref), "cache trace differs from the oracle's LRU"
        hits = int(ref[:, 3].sum())
        cpu = int((ref[:, 4] < 0).sum())
        print(f"  trace ok: {len(ref)} accesses, hit rate {hits / max(len(ref), 1):.3f}, fills {dl.n_fills}, "
              f"cpu runs {dl.cpu_runs}, waves>1 in {int((ref[:, 6] > 0).sum())} accesses, "
              f"{n_checked} layer-step outputs checked", flush=True)
        assert dl.n_fills == len(ref) - hits - cpu
        assert dl.cpu_runs == cpu
        assert cpu_left <= 0 or not cpu_layers, "no CPU-run layer-step was output-checked"
        return ref
    finally:
        store.close()


def epoch_samples(cfg, steps, per_epoch, seed):
    """(step, layer) output checks: the first step of every epoch (the bias has just been re-drawn) and
    `per_epoch` seeded steps inside each epoch, each at a seeded layer."""
    r = np.random.default_rng(seed)
    epoch = cfg.epoch or steps
    out = set()
    for e0 in range(0, steps, epoch):
        e1 = min(e0 + epoch, steps)
        out.add((e0, int(r.integers(0, cfg.L))))
        for st in r.choice(np.arange(e0 + 1, e1), size=min(per_epoch, e1 - e0 - 1), replace=False):
            out.add((int(st), int(r.integers(0, cfg.L))))
    return out


@pytest.mark.parametrize("native", [True, False], ids=["driver", "python"])
def test_tiny_fp32_all_steps(native):
    cfg = CONFIGS["tiny_f32_h256_e16"]
    ref = run_decode(cfg, cfg.steps, set(), check_all_outputs=True, native=native)
    assert (ref[:, 6] > 0).any(), "the tiny config should exercise multi-wave layer-steps"


@pytest.mark.timeout(600)
def test_decode_bf16_full():
    cfg = CONFIGS["decode_bf16_h4096_e256"]
    run_decode(cfg, cfg.steps, {(s, 0) for s in (0, 1, 2, 63, 255, 511, 767, 1023)})


@pytest.mark.timeout(900)
def test_stack48_bf16_full():
    """All 512 steps of the 48-layer stack: routing, grouping and the whole cache trace bit-exact across the
    bias re-draws at steps 128, 256 and 384, outputs sampled in every epoch (including its first step)."""
    cfg = CONFIGS["stack48_bf16_h2048_e128"]
    sample = epoch_samples(cfg, cfg.steps, 2, seed=3)
    ref = run_decode(cfg, cfg.steps, sample)
    for e0 in range(0, cfg.steps, cfg.epoch):
        ep = ref[(ref[:, 0] >= e0) & (ref[:, 0] < e0 + cfg.epoch)]
        print(f"  epoch from step {e0}: miss rate {1 - ep[:, 3].mean():.4f} over {len(ep)} accesses", flush=True)


@pytest.mark.timeout(900)
def test_decode_int4_full():
    cfg = CONFIGS["decode_int4_t8_l8"]
    run_decode(cfg, cfg.steps, {(0, 0), (100, 0), (255, 0), (1, 5), (128, 5), (254, 5)})


@pytest.mark.timeout(900)
def test_decode_mxfp4_full():
    cfg = CONFIGS["decode_mxfp4_t8_l8"]
    run_decode(cfg, cfg.steps, {(0, 0), (100, 0), (255, 0), (1, 5), (128, 5), (254, 5)})


@pytest.mark.parametrize("native", [True, False], ids=["driver", "python"])
def test_resize_small_all_outputs(native):
    """The cache shrinks (entries above the new size move), then grows into a new buffer; every output and
    the whole trace against the oracle."""
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name="resize_small", L=3, T=3, H=256, I=128, E=16,
                              k=2, zipf_s=1.2, epoch=8, S=10)
    run_decode(cfg, 36, set(), check_all_outputs=True, native=native, resizes={12: 4, 24: 14})


def fused_small(I):
    """Single-token bf16 steps whose down projection forms the output when every expert is resident (6 slots
    for 16 experts: steps with and without misses alternate)."""
    return dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name=f"fused_small_i{I}", L=2, T=1, H=256, I=I,
                               E=16, k=4, zipf_s=1.0, epoch=10, S=6)


@pytest.mark.parametrize("I", [512, 1024, 1536, 2048])
def test_fused_combine_all_outputs(I):
    """Every output of 40 steps x 2 layers against the oracle, for each fragment share per wave (I / 512)."""
    cfg = fused_small(I)
    ref = run_decode(cfg, 40, set(), check_all_outputs=True)
    assert (ref[:, 3] == 0).sum() > 10 and (ref[:, 3] == 1).sum() > 40


def test_fused_combine_resize_all_outputs():
    """The fused path across a shrink and a grow into a new buffer (the slot table copy is uploaded again)."""
    cfg = fused_small(512)
    run_decode(cfg, 36, set(), check_all_outputs=True, resizes={12: 3, 24: 8})


@pytest.mark.parametrize("case", ["fused", "tokens3"])
def test_invalidate_between_steps_all_outputs(case):
    """Keys unmapped between steps (moe_cache_invalidate): the GPU copy of the slot table is uploaded again
    before the next step lists its resident experts; every output and the trace against the oracle."""
    cfg = fused_small(1024) if case == "fused" else dataclasses.replace(
        CONFIGS["decode_bf16_h4096_e256"], name="inval_small", L=2, T=3, H=256, I=128, E=16, k=2, zipf_s=1.2,
        epoch=8, S=10)
    run_decode(cfg, 30, set(), check_all_outputs=True, invalidate={6: 1, 13: 3, 21: 2})


def test_fused_combine_split_all_outputs():
    """Single-token steps with misses divided 1:3 between fills and the CPU: steps with every expert resident
    take the fused combine, the rest the combine kernel after the CPU rows; every output checked."""
    cfg = fused_small(1024)
    ref = run_decode(cfg, 40, set(), check_all_outputs=True, split=(1, 3))
    assert (ref[:, 4] < 0).sum() > 5 and (ref[:, 3] == 1).sum() > 40


def test_fused_combine_bf16_output():
    """Two identical decoders over one pool, one writing fp32 outputs and one bf16: the bf16 output is the
    fp32 one rounded to nearest even, on steps with every expert resident (fused combine) and with misses
    (combine kernel) alike."""
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import DecodeLayer
    cfg = fused_small(2048)
    store = make_store(cfg)
    try:
        A = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
        B = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
        Wr = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        ob = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
        s = torch.cuda.current_stream()
        misses = 0
        for step in range(30):
            for layer in range(cfg.L):
                b = gen.router_bias(cfg, layer, step, dev)
                x = gen.tokens(cfg, step, layer, dev)
                oa = A.step(step, layer, x, Wr[layer], b)
                misses += L.moe_decoder_step(B.dec, step, layer, x, Wr[layer], b, ob, s)
                torch.cuda.synchronize()
                assert torch.equal(ob, oa.to(torch.bfloat16)), f"step {step} layer {layer}"
        assert 0 < misses < 30 * cfg.L * cfg.k
    finally:
        store.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wfmt", ["bf16", "int4", "mxfp4"])
def test_split_small_all_outputs(wfmt):
    """Misses divided 1:3 between GPU fills and CPU execution; every output checked."""
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name=f"split_small_{wfmt}", L=3, T=4, H=512, I=256,
                              E=32, k=4, zipf_s=1.0, S=8, wfmt=wfmt)
    ref = run_decode(cfg, 24, set(), check_all_outputs=True, split=(1, 3))
    assert (ref[:, 4] < 0).sum() > 10 and (ref[:, 3] == 0).sum() > (ref[:, 4] < 0).sum()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", ["tiny_waves", "split_small", "fused"])
def test_poisoned_fills_all_outputs(case, monkeypatch):
    """Debug mode: every fill first sets its victim slot to 0xFF bytes (NaN in every weight format), so a kernel
    that read a slot before its copy landed, or a copy that overwrote a slot still being read, would give
    non-finite or wrong outputs. Every output of multi-wave layer-steps (the hits' FFN overlapping the copies)
    and of split layer-steps is checked."""
    monkeypatch.setenv("MOE_DEBUG_POISON_FILLS", "1")
    if case == "tiny_waves":
        cfg = CONFIGS["tiny_f32_h256_e16"]
        ref = run_decode(cfg, 32, set(), check_all_outputs=True)
        assert (ref[:, 6] > 0).any()
    elif case == "split_small":
        cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name="split_small", L=3, T=4, H=512, I=256,
                                  E=32, k=4, zipf_s=1.0, S=8)
        ref = run_decode(cfg, 16, set(), check_all_outputs=True, split=(1, 3))
        assert (ref[:, 4] < 0).any()
    else:  # single-token steps whose down projection forms the output
        ref = run_decode(fused_small(1024), 24, set(), check_all_outputs=True)
        assert (ref[:, 3] == 0).any()


@pytest.mark.timeout(600)
def test_stack48_split_cut():
    """The 48-layer stack with misses divided in the ratio of a measured fill and CPU rate (56 : 165 GB/s)."""
    cfg = CONFIGS["stack48_bf16_h2048_e128"]
    run_decode(cfg, 10, {(9, 47)}, split=(56, 165), cpu_check=(4, (0, 1, 2)))


def oracle_group_rows(x64, perm_src, offsets, rows, get_expert):
    """Oracle rows of y_perm (row r = the output of r's expert for token perm_src[r]), evaluated one expert
    at a time over all requested rows of its group. Returns (sorted unique rows, values)."""
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    y = np.zeros((len(rows), x64.shape[1]))
    for e in np.unique(e_of):
        sel = e_of == e
        y[sel] = oracle.swiglu_expert(x64[perm_src[rows[sel]]], *get_expert(e))
    return rows, y


class LayerCopy:
    """Device copies of one prefill layer's routing, y_perm and output, taken on the stream right after the
    layer, so that later layers can reuse the buffers before anything is read on the host."""

    def __init__(self, pl, T):
        rb = pl.rb
        self.idx, self.w = rb.topk_idx[:T].clone(), rb.topk_w[:T].clone()
        self.counts, self.offsets = rb.counts.clone(), rb.offsets.clone()
        self.perm_src, self.perm_pos = rb.perm_src[:T * pl.k].clone(), rb.perm_pos[:T].clone()
        self.y_perm, self.out = pl.y_perm[:T * pl.k].clone(), pl.out[:T].clone()


def prefill_check(cfg, layer, got, x, Wr, b, n_tokens=None, tile_rows=256):
    """Routing and grouping of every token; outputs of every token (n_tokens None) or of a seeded sample of
    n_tokens tokens plus the tokens of the largest and smallest groups; and the y_perm rows of the first and
    last `tile_rows`-row tile of the largest group and of every row of one group whose size is not a multiple
    of 128 (a partial tile). The oracle evaluates each expert once over all requested rows of its group."""
    T, k = cfg.T, cfg.k
    l64 = oracle.router_logits(x, Wr, b)
    idx = npi(got.idx)
    check_routing(idx, np64(got.w), l64, k)
    counts, offsets, perm_pos, perm_src = check_permutation(idx, npi(got.counts), npi(got.offsets),
                                                            npi(got.perm_src), npi(got.perm_pos), cfg.E)
    if n_tokens is None:
        tokens = np.arange(T)
    else:
        r = np.random.default_rng(1000 + layer)
        tokens = list(r.choice(T, n_tokens, replace=False))
        for e in (int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))):
            tokens.append(int(np.nonzero((idx == e).any(1))[0][0]))
        tokens = np.unique(np.asarray(tokens))
    rows = [perm_pos[tokens].reshape(-1)]
    big = int(np.argmax(counts))
    c0, o0 = int(counts[big]), int(offsets[big])
    last = o0 + (c0 - 1) // tile_rows * tile_rows
    rows += [np.arange(o0, o0 + min(tile_rows, c0)), np.arange(last, o0 + c0)]
    partial = [e for e in np.argsort(-counts) if counts[e] > 0 and counts[e] % 128 != 0 and e != big]
    if partial:
        e = int(partial[0])
        rows.append(np.arange(offsets[e], offsets[e] + counts[e]))
    x64 = np64(x)
    ge = ExpertCache64(cfg, layer, cap=8)
    rr, yref = oracle_group_rows(x64, perm_src, offsets, np.concatenate(rows), ge)
    y_got = np64(got.y_perm[torch.as_tensor(rr, device=got.y_perm.device)])
    check_close(y_got, yref, f"{cfg.name} layer {layer}: {len(rr)} y_perm rows")
    # outputs of the sampled tokens from the oracle's rows on the GPU's selection
    pos = {int(r_): n for n, r_ in enumerate(rr)}
    w = oracle.topk_weights(l64[tokens], idx[tokens])
    out_ref = np.zeros((len(tokens), cfg.H))
    for j in range(k):
        out_ref += w[:, j:j + 1] * yref[[pos[int(p)] for p in perm_pos[tokens, j]]]
    out_got = np64(got.out[torch.as_tensor(tokens, device=got.out.device)])
    check_close(out_got, out_ref, f"{cfg.name} layer {layer}: {len(tokens)} token outputs")
    part = f" + partial group of {counts[partial[0]]}" if partial else ""
    print(f"  layer {layer}: {len(tokens)} tokens and {len(rr)} y_perm rows match (largest group {c0} rows, "
          f"first and last tile{part}); active experts {int((counts > 0).sum())}", flush=True)
    return counts


def pack_resident(cfg, wf):
    from routed_expert_layer_amd import _lib as L
    blob = L.moe_expert_bytes(wf, cfg.H, cfg.I)
    stride = (blob + 4095) // 4096 * 4096
    buf = torch.empty(cfg.E * stride, dtype=torch.uint8, device=dev)
    for e in range(cfg.E):
        if wf == L.MOE_W_MXFP4:
            w = gen.expert_mxfp4(cfg, 0, e, dev)
            L.moe_pack_expert(wf, cfg.H, cfg.I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"],
                              buf[e * stride:])
        else:
            W1, W3, W2 = gen.expert_weights(cfg, 0, e, dev)
            L.moe_pack_expert(wf, cfg.H, cfg.I, W1, W3, W2, None, None, None, buf[e * stride:])
    return buf, stride


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_bf16_t4096_e256", "prefill_mxfp4_t4096_e256"])
def test_prefill_4096_every_token(name):
    """The 4096-token chunk with all experts resident, one moe_prefill_layer call: every token's output and
    every y_perm row against the oracle."""
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import PrefillLayer
    cfg = CONFIGS[name]
    wf = L.MOE_W_MXFP4 if cfg.wfmt == "mxfp4" else L.MOE_W_BF16
    print(f"prefill {cfg.name}: T={cfg.T}, every token", flush=True)
    buf, stride = pack_resident(cfg, wf)
    pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, stride, dev, keep_logits=True, wfmt=wf)
    Wr = gen.router_weight(cfg, 0, dev)
    b = gen.router_bias(cfg, 0, 0, dev)
    x = gen.tokens(cfg, 0, 0, dev)
    pl.forward(x, Wr, b, buf)
    got = LayerCopy(pl, cfg.T)
    torch.cuda.synchronize()
    counts = prefill_check(cfg, 0, got, x, Wr, b, n_tokens=None)  # every token, so every y_perm row
    print(f"  tokens per expert: min {counts.min()} max {counts.max()} mean {counts.mean():.1f}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_db_bf16_t16384_l8", "prefill_db_mxfp4_t16384_l8"])
def test_prefill_16384_double_buffered(name):
    """Eight 16384-token layers through the double buffer, enqueued back to back with no host wait: layer
    l+2's copy into the buffer layer l read must wait for layer l's compute (the pipe's ordering), or the
    outputs of layer l would be computed from the wrong weights. Each layer's results are copied on the stream
    and all are checked at the end: routing of every token, 1024 sampled token outputs and the tile rows."""
    from routed_expert_layer_amd import _lib as L
    from routed_expert_layer_amd.runtime import PrefillLayer
    cfg = CONFIGS[name]
    store = make_store(cfg)
    try:
        pipe = L.MoePipe(store.layer_ptrs, store.layer_bytes)
        pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, store.stride, dev, keep_logits=True, wfmt=store.wfmt)
        s = torch.cuda.current_stream()
        xs = [gen.tokens(cfg, 0, layer, dev) for layer in range(cfg.L)]
        Wrs = [gen.router_weight(cfg, layer, dev) for layer in range(cfg.L)]
        bs = [gen.router_bias(cfg, layer, 0, dev) for layer in range(cfg.L)]
        torch.cuda.synchronize()
        got = []
        for layer in range(cfg.L):
            base = L.moe_pipe_begin_layer(pipe, layer, s)
            pl.forward(xs[layer], Wrs[layer], bs[layer], base, stream=s)
            L.moe_pipe_end_layer(pipe, layer, s)
            got.append(LayerCopy(pl, cfg.T))
        print(f"  {cfg.L} layers enqueued", flush=True)
        torch.cuda.synchronize()
        # 1024 tokens per layer with bf16 experts; fewer with MXFP4, whose oracle weights cost more to form
        n_tok = 1024 if cfg.wfmt == "bf16" else 256
        for layer in range(cfg.L):
            prefill_check(cfg, layer, got[layer], xs[layer], Wrs[layer], bs[layer], n_tokens=n_tok)
            print(f"    copy {L.moe_pipe_copy_ms(pipe, layer):.1f} ms", flush=True)
        pipe.close()
    finally:
        store.close()
