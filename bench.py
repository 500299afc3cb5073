#!/usr/bin/env python3
"""Throughput of the routed expert layer on one MI355X.

Default workload: one-layer bf16 decode, batch 1 token per step, hidden 4096,
256 routed experts (SwiGLU intermediate 2048), top-6, Zipf(1.1)-biased router,
64 expert slots in HBM, the full expert pool in page-locked host memory and
misses filled before compute. A step is one pass of the whole path over one
token: route (logits, top-k, grouping), host LRU resolve, fills of misses,
grouped expert FFN, combine. Warm-up steps are the first W steps of the
trace; the next K steps are timed.

Also reported: the dominant kernel (the decode expert FFN) against the HBM
roofline, timed with HIP events on its own stream; the pinned host-to-device
fill bandwidth; the 4096-token prefill layer's expert GEMM against the bf16
matrix-core peak; the 8-layer 16384-token prefill with double-buffered layer
copies (GEMM TFLOP/s, copy GB/s, how much compute the copies hide); the
int4 8-layer decode and the 48-layer bf16 decode stack (tokens/s, FFN GB/s,
hit rate); and the CPU oracle on a bounded sample of the decode workload.

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
PEAK_CLOCK_GHZ = 2.4         # the clock the matrix-core peak is quoted at
PCIE_PEAK_GBS = 63.0         # PCIe Gen5 x16, one direction


class EventTimer:
    """Pairs of HIP events recorded on the stream the timed kernels run on."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        self.work = []
        self.i = 0
        self.enabled = False

    def begin(self, s):
        if self.enabled and self.i < len(self.ev):
            self.ev[self.i][0].record(s)

    def end(self, s, work):
        if self.enabled and self.i < len(self.ev):
            self.ev[self.i][1].record(s)
            self.work.append(work)
            self.i += 1

    def result(self):
        ms = [a.elapsed_time(b) for a, b in self.ev[:self.i]]
        return sum(self.work), sum(ms), len(ms)


def _definition(src, signature):
    """Text of the definition that starts at `signature` (through its matching closing brace)."""
    i = src.index(signature)
    j = src.index("{", i)
    depth = 0
    for n in range(j, len(src)):
        if src[n] == "{":
            depth += 1
        elif src[n] == "}":
            depth -= 1
            if depth == 0:
                return src[i:n + 1]
    raise ValueError(signature)


def decode_ffn_digest(root):
    """sha256 over the source text the decode expert-FFN kernels are built from: both kernels, their
    wave loop, launchers, the work sources, the device helpers they call and the work-list / blob-layout
    definitions."""
    import hashlib
    csrc = os.path.join(root, "routed_expert_layer_amd", "csrc")
    ffn = open(os.path.join(csrc, "kernels_ffn.hip")).read()
    hdr = open(os.path.join(csrc, "moe_kernels.hpp")).read()
    dev = open(os.path.join(csrc, "dev_common.hpp")).read()
    # the device helpers those kernels use: vector types, bf16 rounding, SiLU, loads, the bf16 product
    helpers = [line for line in dev.splitlines() if line.startswith("typedef")]
    helpers += [_definition(dev, sig) for sig in ("uint16_t f32_to_bf16(", "float silu(", "u32x4_t ld16(",
                                                  "u32x4_t ld16_nt(", "f32x4_t mfma_bf16(")]
    parts = ["\n".join(helpers),
             _definition(ffn, "__global__ __launch_bounds__(256) void ffn1_decode_bf16("),
             _definition(ffn, "__global__ __launch_bounds__(256) void ffn2_decode_bf16("),
             _definition(ffn, "__global__ __launch_bounds__(1024) void ffn2_combine_bf16("),
             ffn[ffn.index("constexpr int kFuseWaves ="):].split("\n", 1)[0],
             _definition(ffn, "bool ffn_combine_ok("), _definition(ffn, "hipError_t ffn_combine_kernels("),
             _definition(ffn, "hipError_t launch_ffn_decode_combine("),
             _definition(ffn, "hipError_t launch_ffn_decode("),
             _definition(ffn, "hipError_t launch_ffn_decode_dev("),
             _definition(ffn, "hipError_t decode_kernels("), _definition(ffn, "struct ArgWork"),
             _definition(ffn, "struct DevList"), _definition(ffn, "struct DevHits"),
             _definition(ffn, "struct DevWork"), _definition(ffn, "f32x4_t bf16_wave_dot("),
             _definition(ffn, "struct PlainLoad"), _definition(ffn, "void bf16_ffn1_tile("),
             _definition(ffn, "void bf16_ffn2_tile("),
             _definition(ffn, "void st16("), ffn[ffn.index("constexpr int kU ="):].split("\n", 1)[0],
             _definition(hdr, "struct WorkArgs"), _definition(hdr, "inline BlobLayout blob_layout("),
             hdr[hdr.index("constexpr int kFuseItems ="):].split("\n", 1)[0]]
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


def measured_traffic(root):
    """HBM bytes per FFN call from the committed counter summary, if the kernels' sources are unchanged since."""
    path = os.path.join(root, "profiles", "decode_ffn_hbm_traffic.json")
    try:
        j = json.load(open(path))
        if j["kernel_source_sha256"] != decode_ffn_digest(root):
            return None
        return int(j["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def section(name):
    """One progress line per bench section (stderr), so a long run shows where it is."""
    print(f"[bench] {name}", file=sys.stderr, flush=True)


def percentile(xs, p):
    xs = sorted(xs)
    if not xs:
        return 0.0
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


def bench_device(torch, cfg, store, Wrs, warm, steps, x_of, b_of):
    """Device-controlled decode (cache control in GPU memory, moe_device_decoder_step): every step is enqueued
    with no host synchronisation, eagerly and as replays of one graph holding all layers of a token step. The
    inputs of all steps are staged in HBM first; each step copies its x (and, when the epoch changes, the
    biases) into the static buffers the graph reads, on the same stream."""
    from routed_expert_layer_amd.runtime import DeviceDecodeLayer
    dev = "cuda"
    n = warm + steps
    x_all = torch.stack([torch.stack([x_of(st, l) for l in range(cfg.L)]) for st in range(n)])
    epoch = cfg.epoch or (n + 1)
    b_all = {ep: torch.stack([b_of(l, ep * epoch) for l in range(cfg.L)]) for ep in sorted({st // epoch
                                                                                           for st in range(n)})}
    cs = torch.cuda.Stream()

    def one(graph):
        dl = DeviceDecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
        xs = torch.empty_like(x_all[0])
        bs = torch.empty_like(next(iter(b_all.values())))
        outs = torch.empty((cfg.L, cfg.T, cfg.H), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def enqueue():
            for l in range(cfg.L):
                dl.step(l, xs[l], Wrs[l], bs[l], cs, out=outs[l])

        g = DeviceDecodeLayer.capture(enqueue, cs) if graph else None

        def run_steps(a, b):
            ep_prev = None
            with torch.cuda.stream(cs):
                for st in range(a, b):
                    xs.copy_(x_all[st], non_blocking=True)
                    if st // epoch != ep_prev:
                        ep_prev = st // epoch
                        bs.copy_(b_all[ep_prev], non_blocking=True)
                    if g is not None:
                        DeviceDecodeLayer.replay(g, cs)
                    else:
                        enqueue()

        run_steps(0, warm)
        h0, m0, _ = dl.stats()
        t0 = time.perf_counter()
        run_steps(warm, n)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        h1, m1, _ = dl.stats()
        if g is not None:
            g.close()
        return dict(tokens_per_s=steps * cfg.T / el, ms_per_step=el * 1e3 / steps,
                    hit_rate=(h1 - h0) / max(h1 - h0 + m1 - m0, 1), fills_timed=m1 - m0)

    return dict(eager=one(False), graph=one(True))


def decode_variants(args, torch, cfg, store, Wr, xs, bias):
    """The one-layer decode workload with the pages' adaptive misses (misses divided between fills and CPU
    execution in the ratio of the measured fill and CPU rates) and with the cache control in GPU memory."""
    from routed_expert_layer_amd.runtime import DecodeLayer
    dev = "cuda"
    s = torch.cuda.current_stream()
    n_total = args.warmup + args.steps
    dl2 = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
    rates = [int(r) for r in dl2.measure_rates()]
    dl2.set_split(*rates)
    for step in range(args.warmup):
        dl2.step(step, 0, xs[step], Wr, bias(step), s)
    torch.cuda.synchronize()
    f2, c2 = dl2.n_fills, dl2.cpu_runs
    lat2 = []
    t2 = prev = time.perf_counter()
    for step in range(args.warmup, n_total):
        dl2.step(step, 0, xs[step], Wr, bias(step), s)
        now = time.perf_counter()
        lat2.append(now - prev)
        prev = now
    torch.cuda.synchronize()
    el2 = time.perf_counter() - t2
    tr2 = dl2.trace()
    tm2 = tr2[tr2[:, 0] >= args.warmup]
    split = dict(tokens_per_s=args.steps * cfg.T / el2, ms_per_step=el2 * 1e3 / args.steps,
                 step_ms_p50=percentile(lat2, 50) * 1e3, hit_rate=float(tm2[:, 3].mean()) if len(tm2) else 0.0,
                 fills_timed=dl2.n_fills - f2, cpu_runs_timed=dl2.cpu_runs - c2, split_rates_mbs=rates)
    del dl2
    device = bench_device(torch, cfg, store, [Wr], args.warmup, args.steps, lambda st, l: xs[st],
                          lambda l, st: bias(st))
    return split, device


def full_trace(args, torch, L, cfg, store, Wr, xs, bias, split=False):
    """Every step of the one-layer decode workload from a cold cache (whatever --steps/--warmup say): tokens/s,
    fills, hit rate and per-step latency percentiles over the whole trace, fills included. With split, misses
    are divided between fills and CPU execution in the ratio of the rates measured on this machine."""
    from routed_expert_layer_amd.runtime import DecodeLayer
    dev = "cuda"
    s = torch.cuda.current_stream()
    from workloads import gen
    n = cfg.steps
    x_all = [xs[st] if st < len(xs) else gen.tokens(cfg, st, 0, dev) for st in range(n)]
    dl = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
    rates = None
    if split:
        rates = [int(r) for r in dl.measure_rates()]
        dl.set_split(*rates)
    torch.cuda.synchronize()
    lat = []
    t0 = prev = time.perf_counter()
    for st in range(n):
        dl.step(st, 0, x_all[st], Wr, bias(st), s)
        now = time.perf_counter()
        lat.append(now - prev)
        prev = now
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    lat[-1] += time.perf_counter() - prev
    tr = dl.trace()
    return dict(steps=n, tokens_per_s=n * cfg.T / el, ms_per_step=el * 1e3 / n, fills=int(dl.n_fills),
                cpu_runs=int(dl.cpu_runs), hit_rate=float(tr[:, 3].mean()),
                step_ms_p50=percentile(lat, 50) * 1e3, step_ms_p99=percentile(lat, 99) * 1e3,
                step_ms_max=max(lat) * 1e3, split_rates_mbs=rates)


def mall_flushed_roofline(torch, L, dl, cfg, store, x, reps=40):
    """The decode expert FFN of six resident experts, one call at a time with the last-level cache (256 MB)
    flushed before each: a 512 MB buffer is written on the stream between calls, so the experts' 302 MB come
    from HBM. HIP events around each call on the stream it runs on; the same calls back to back (experts warm
    in that cache) for comparison."""
    import numpy as np
    dev = "cuda"
    s = torch.cuda.current_stream()
    keys = [k for k in range(cfg.E) if L.moe_cache_slot_of(dl.cache, k) >= 0][:cfg.k]
    if len(keys) < cfg.k:
        return None
    work = np.array([[k, L.moe_cache_slot_of(dl.cache, k), j, 1] for j, k in enumerate(keys)], np.int32)
    perm_src = torch.zeros(cfg.k, dtype=torch.int32, device=dev)
    y = torch.empty((cfg.k, cfg.H), dtype=torch.float32, device=dev)
    ws = torch.empty(L.moe_ffn_workspace_size(cfg.k, cfg.H, cfg.I, store.wfmt), dtype=torch.uint8, device=dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    alg = len(keys) * store.blob + cfg.k * (cfg.H * 2 + 2 * cfg.I * 2 + cfg.H * 4)

    def run(flush):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps + 3):
            if flush:
                scratch.fill_(i & 0xFF)
            if i >= 3:
                ev[i - 3][0].record(s)
            L.moe_ffn(x, perm_src, work, dl.slots, store.stride, store.wfmt, cfg.H, cfg.I, y, ws, L.MOE_FFN_DECODE, s)
            if i >= 3:
                ev[i - 3][1].record(s)
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / reps
        return us

    us_f, us_w = run(True), run(False)
    del scratch
    return dict(kernel="ffn1_decode_bf16 + ffn2_decode_bf16, six resident experts, one call at a time",
                algorithmic_bytes_per_launch=alg, launches=reps,
                flushed=dict(avg_launch_us=round(us_f, 2), achieved_gbs=round(alg / us_f / 1e3, 1),
                             frac=round(alg / us_f / 1e3 / HBM_PEAK_GBS, 4)),
                cache_warm=dict(avg_launch_us=round(us_w, 2), achieved_gbs=round(alg / us_w / 1e3, 1),
                                frac=round(alg / us_w / 1e3 / HBM_PEAK_GBS, 4)))


def bench_decode(args, torch, L, gen, cfg):
    from routed_expert_layer_amd.runtime import DecodeLayer, ExpertStore
    dev = "cuda"
    t0 = time.time()
    store = ExpertStore(cfg.L, cfg.E, cfg.H, cfg.I, cfg.wfmt, phys_layers=cfg.pool_layers)
    for layer in range(store.P):
        store.pack_layer(layer, lambda e: gen.expert_weights(cfg, layer, e, dev))
    print(f"[bench] pool {store.nbytes / 1e9:.2f} GB packed in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    n_total = args.warmup + args.steps
    xs = [gen.tokens(cfg, s, 0, dev) for s in range(n_total)]
    Wr = gen.router_weight(cfg, 0, dev)
    biases = {}
    dl = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
    s = torch.cuda.current_stream()

    def bias(step):
        ep = (step // cfg.epoch) if cfg.epoch else 0
        if ep not in biases:
            biases[ep] = gen.router_bias(cfg, 0, step, dev)
        return biases[ep]

    for step in range(args.warmup):
        dl.step(step, 0, xs[step], Wr, bias(step), s)
    torch.cuda.synchronize()
    fills0 = dl.n_fills
    # HIP events around the expert-FFN calls of no-fill steps, on stream s: every 8th in long runs (the events
    # then barely touch the step time), every one in short runs (so the sample is not a handful of calls)
    L.moe_decoder_profile(dl.dec, 8 if args.steps > 256 else 1)
    lat = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    prev = t_start
    for step in range(args.warmup, n_total):
        dl.step(step, 0, xs[step], Wr, bias(step), s)
        now = time.perf_counter()
        lat.append(now - prev)
        prev = now
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    lat[-1] += time.perf_counter() - prev
    ffn_bytes, ffn_ms, n_ffn = L.moe_decoder_ffn_stats(dl.dec)
    L.moe_decoder_profile(dl.dec, False)
    trace = dl.trace()
    timed = trace[trace[:, 0] >= args.warmup]
    hit_rate = float(timed[:, 3].mean()) if len(timed) else 0.0
    # steps that needed no fill: the layer's throughput without PCIe in the step. A step's host-side
    # interval ends when its counts reach the host, which waits for the previous step's FFN and fills:
    # a fill in step t shows in the interval of step t + 1, so both are left out.
    miss_steps = set(int(v) for v in timed[timed[:, 3] == 0][:, 0])
    hit_lat = [lat[i] for i in range(len(lat))
               if args.warmup + i not in miss_steps and args.warmup + i - 1 not in miss_steps]
    no_fill_tps = cfg.T * len(hit_lat) / sum(hit_lat) if hit_lat else 0.0

    split = device = None
    if not args.no_variants:
        split, device = decode_variants(args, torch, cfg, store, Wr, xs, bias)

    full = full_trace(args, torch, L, cfg, store, Wr, xs, bias)
    if not args.no_variants:
        full["cpu_split"] = full_trace(args, torch, L, cfg, store, Wr, xs, bias, split=True)
    flushed = mall_flushed_roofline(torch, L, dl, cfg, store, xs[0])

    # pinned host -> HBM fill bandwidth: blobs copied on the fill stream
    fs = dl.fill_stream
    n_copy = min(16, cfg.S)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(fs)
    misses = [[key, slot, -1, 0] for slot, key in enumerate(range(n_copy))]
    L.cache_fill_async(dl.cache, misses, store.layer_ptrs, store.stride, store.blob, dl.slots, store.stride, fs, fs)
    e1.record(fs)
    torch.cuda.synchronize()
    fill_gbs = n_copy * store.blob / (e0.elapsed_time(e1) * 1e-3) / 1e9
    store.close()
    return dict(
        value=args.steps * cfg.T / elapsed,
        ms_per_step=elapsed * 1e3 / args.steps,
        ffn=dict(bytes=ffn_bytes, ms=ffn_ms, n=n_ffn),
        decode=dict(tokens_per_s_no_fill_steps=no_fill_tps, no_fill_steps=len(hit_lat),
                    step_ms_p50=percentile(lat, 50) * 1e3, step_ms_p99=percentile(lat, 99) * 1e3,
                    step_ms_max=max(lat) * 1e3, hit_rate=hit_rate, fills_timed=dl.n_fills - fills0,
                    fills_warmup=fills0, fill_gbs=fill_gbs, fill_frac_pcie=fill_gbs / PCIE_PEAK_GBS,
                    pool_gb=store.nbytes / 1e9, slots=cfg.S, cpu_split=split, device_control=device,
                    full_trace=full),
        roofline_mall_flushed=flushed,
    )


class ClockRecord:
    """Mean shader clock of the prefill expert GEMMs enqueued while it is active (moe_clock_record)."""

    def __init__(self, torch, L):
        self.L = L
        self.sums = torch.zeros(2, dtype=torch.int64, device="cuda")

    def __enter__(self):
        self.L.moe_clock_record(self.sums)
        return self

    def __exit__(self, *exc):
        self.L.moe_clock_record(None)

    def ghz(self):
        cyc, ticks = (int(v) for v in self.sums.cpu())
        return cyc / ticks / 10.0 if ticks > 0 else None


GROUP_BINS = [1, 2, 17, 65, 129, 257, 1025, 4097, 1 << 31]  # rows per active expert: 1, 2-16, 17-64, ...


def group_stats(counts):
    """Tokens per active expert of a layer (or several): percentiles and a coarse histogram."""
    import numpy as np
    c = np.asarray(counts).reshape(-1)
    c = c[c > 0]
    if c.size == 0:
        return dict(active=0)
    hist = np.histogram(c, bins=GROUP_BINS)[0]
    labels = [f"{a}" if b == a + 1 else f"{a}-{b - 1}" if b < (1 << 31) else f">={a}"
              for a, b in zip(GROUP_BINS[:-1], GROUP_BINS[1:])]
    return dict(active=int(c.size), min=int(c.min()), p10=float(np.percentile(c, 10)),
                p50=float(np.percentile(c, 50)), p90=float(np.percentile(c, 90)), max=int(c.max()),
                histogram={lab: int(n) for lab, n in zip(labels, hist) if n})


def at_clock(tfs, ghz):
    """Share of the matrix-core peak scaled to the measured clock."""
    return tfs / (MFMA_BF16_PEAK_TFS * ghz / PEAK_CLOCK_GHZ) if ghz else None


def bench_prefill(args, torch, L, gen, cfg, reps=5):
    from routed_expert_layer_amd.runtime import PrefillLayer
    dev = "cuda"
    wf = L.MOE_W_MXFP4 if cfg.wfmt == "mxfp4" else L.MOE_W_BF16
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
    pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, stride, dev, wfmt=wf)
    Wr = gen.router_weight(cfg, 0, dev)
    b = gen.router_bias(cfg, 0, 0, dev)
    x = gen.tokens(cfg, 0, 0, dev)
    s = torch.cuda.current_stream()
    for _ in range(2):
        pl.forward(x, Wr, b, buf, s)
    # the whole layer (one moe_prefill_layer call: routing, the work list planned on the GPU, the grouped GEMM,
    # the combine), then the grouped GEMM alone on the same routing, each timed with events on the stream
    lay = EventTimer(torch, reps)
    lay.enabled = True
    timer = EventTimer(torch, reps)
    timer.enabled = True
    torch.cuda.synchronize()
    for _ in range(reps):
        lay.begin(s)
        pl.forward(x, Wr, b, buf, s)
        lay.end(s, 0)
    with ClockRecord(torch, L) as clk:
        for _ in range(reps):
            timer.begin(s)
            pl.ffn(x, buf, stream=s)
            timer.end(s, 6.0 * cfg.H * cfg.I * cfg.T * cfg.k)
        torch.cuda.synchronize()
    _, lay_ms, _ = lay.result()
    flops, ms, n = timer.result()
    counts = pl.rb.counts.cpu().numpy()
    active = int((counts > 0).sum())
    tfs = flops / (ms * 1e-3) / 1e12
    wbytes = active * blob
    del buf
    return dict(workload=cfg.name, tokens=cfg.T, layer_ms=lay_ms / reps, gemm_ms=ms / n, tflops=tfs,
                mfma_frac=tfs / MFMA_BF16_PEAK_TFS, gemm_clock_ghz=clk.ghz(), mfma_frac_at_clock=at_clock(tfs, clk.ghz()),
                weight_gbs=wbytes / (ms / n * 1e-3) / 1e9,
                hbm_frac=wbytes / (ms / n * 1e-3) / 1e9 / HBM_PEAK_GBS, active_experts=active,
                group_min=int(counts[counts > 0].min()), group_max=int(counts.max()),
                tokens_per_expert=group_stats(counts))


def bench_prefill_pipeline(args, torch, L, gen, cfg):
    """8-layer prefill: layer l+1's experts copy host -> HBM while layer l computes."""
    from routed_expert_layer_amd.runtime import ExpertStore, PrefillLayer
    dev = "cuda"
    store = ExpertStore(cfg.L, cfg.E, cfg.H, cfg.I, cfg.wfmt, phys_layers=cfg.pool_layers)
    try:
        mx = cfg.wfmt == "mxfp4"
        for layer in range(store.P):
            store.pack_layer(layer, (lambda e: gen.expert_mxfp4(cfg, layer, e, dev)) if mx else
                             (lambda e: gen.expert_weights(cfg, layer, e, dev)))
        xs = [gen.tokens(cfg, 0, l, dev) for l in range(cfg.L)]
        Wrs = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        bs = [gen.router_bias(cfg, l, 0, dev) for l in range(cfg.L)]
        wf = store.wfmt
        pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, store.stride, dev, wfmt=wf)
        s = torch.cuda.current_stream()
        # warm-up pass (kernels and the copy path), then the timed pass
        clk = ClockRecord(torch, L)
        for rep in range(2):
            pipe = L.MoePipe(store.layer_ptrs, store.layer_bytes)
            timer = EventTimer(torch, cfg.L)
            timer.enabled = rep == 1
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cfg.L)]
            layer_counts = []
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if rep == 1:
                clk.__enter__()
            for l in range(cfg.L):
                base = L.moe_pipe_begin_layer(pipe, l, s)
                ev[l][0].record(s)
                # warm-up: one moe_prefill_layer call per layer; timed pass: the same three steps as separate
                # calls, with events around the grouped GEMM
                pl.forward(xs[l], Wrs[l], bs[l], base, s, timer=timer if rep == 1 else None)
                ev[l][1].record(s)
                L.moe_pipe_end_layer(pipe, l, s)
                layer_counts.append(pl.rb.counts.clone())  # on the stream: nothing waits for the GPU
            torch.cuda.synchronize()
            layer_counts = [c.cpu().numpy() for c in layer_counts]
            groups = [(int((c > 0).sum()), int(c.max())) for c in layer_counts]
            if rep == 1:
                clk.__exit__()
            wall = (time.perf_counter() - t0) * 1e3
            copy_ms = [L.moe_pipe_copy_ms(pipe, l) for l in range(cfg.L)]
            comp_ms = [a.elapsed_time(b) for a, b in ev]
            pipe.close()
        flops, gemm_ms, n = timer.result()
        tfs = flops / (gemm_ms * 1e-3) / 1e12
        exposed = max(0.0, wall - sum(copy_ms))
        return dict(workload=cfg.name, layers=cfg.L, tokens_per_layer=cfg.T,
                    gemm_tflops=tfs, mfma_frac=tfs / MFMA_BF16_PEAK_TFS, gemm_clock_ghz=clk.ghz(),
                    mfma_frac_at_clock=at_clock(tfs, clk.ghz()), gemm_ms_per_layer=gemm_ms / n,
                    layer_compute_ms=sum(comp_ms) / cfg.L, copy_ms_per_layer=sum(copy_ms) / cfg.L,
                    copy_gbs=store.layer_bytes / (sum(copy_ms) / cfg.L * 1e-3) / 1e9,
                    copy_frac_pcie=store.layer_bytes / (sum(copy_ms) / cfg.L * 1e-3) / 1e9 / PCIE_PEAK_GBS,
                    wall_ms=wall, compute_hidden_frac=1.0 - min(1.0, exposed / max(sum(comp_ms), 1e-9)),
                    prefill_tokens_per_s=cfg.L * cfg.T / (wall * 1e-3) / cfg.L,
                    active_experts=[g[0] for g in groups], max_group=[g[1] for g in groups],
                    tokens_per_expert=group_stats(layer_counts),
                    weight_sets=store.P)
    finally:
        store.close()


def bench_decode_layers(args, torch, L, gen, cfg, warm, steps):
    """Multi-layer decode with one shared cache: every step runs all layers."""
    from routed_expert_layer_amd.runtime import DecodeLayer, ExpertStore
    dev = "cuda"
    store = ExpertStore(cfg.L, cfg.E, cfg.H, cfg.I, cfg.wfmt, phys_layers=cfg.pool_layers)
    try:
        for layer in range(store.P):
            if cfg.wfmt == "int4":
                store.pack_layer(layer, lambda e: gen.expert_int4(cfg, layer, e, dev))
            elif cfg.wfmt == "mxfp4":
                store.pack_layer(layer, lambda e: gen.expert_mxfp4(cfg, layer, e, dev))
            else:
                store.pack_layer(layer, lambda e: gen.expert_weights(cfg, layer, e, dev))
        n = warm + steps
        xs = [[gen.tokens(cfg, st, l, dev) for l in range(cfg.L)] for st in range(n)]
        Wrs = [gen.router_weight(cfg, l, dev) for l in range(cfg.L)]
        bias = {}

        def b(l, st):
            ep = (st // cfg.epoch) if cfg.epoch else 0
            if (l, ep) not in bias:
                bias[(l, ep)] = gen.router_bias(cfg, l, st, dev)
            return bias[(l, ep)]

        s = torch.cuda.current_stream()

        def run(split):
            dl = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
            rates = None
            if split:
                rates = [int(r) for r in dl.measure_rates()]
                dl.set_split(*rates)
            for st in range(warm):
                for l in range(cfg.L):
                    dl.step(st, l, xs[st][l], Wrs[l], b(l, st), s)
            torch.cuda.synchronize()
            f0, c0 = dl.n_fills, dl.cpu_runs
            L.moe_decoder_profile(dl.dec, 8)
            t0 = time.perf_counter()
            for st in range(warm, n):
                for l in range(cfg.L):
                    dl.step(st, l, xs[st][l], Wrs[l], b(l, st), s)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            fb, fms, fn = L.moe_decoder_ffn_stats(dl.dec)
            tr = dl.trace()
            timed = tr[tr[:, 0] >= warm]
            gbs = fb / (fms * 1e-3) / 1e9
            return dict(tokens_per_s=steps * cfg.T / el, ms_per_step=el * 1e3 / steps,
                        ms_per_layer_step=el * 1e3 / (steps * cfg.L), ffn_gbs=gbs, ffn_hbm_frac=gbs / HBM_PEAK_GBS,
                        ffn_us_per_call=fms * 1e3 / max(fn, 1), hit_rate=float(timed[:, 3].mean()),
                        fills_timed=dl.n_fills - f0, cpu_runs_timed=dl.cpu_runs - c0,
                        split_rates_mbs=rates)

        def epochs():
            # the whole workload from a cold cache, every miss filled: the miss rate of each epoch (the router
            # bias is re-drawn at every epoch start) and the end-to-end rate, fills included
            dl = DecodeLayer(store, cfg.S, cfg.T, cfg.k, cfg.act, dev)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for st in range(cfg.steps):
                for l in range(cfg.L):
                    dl.step(st, l, xs[st][l] if st < n else gen.tokens(cfg, st, l, dev), Wrs[l], b(l, st), s)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            tr = dl.trace()
            ep = tr[:, 0] // cfg.epoch
            return dict(steps=cfg.steps, epoch_steps=cfg.epoch, tokens_per_s=cfg.steps * cfg.T / el,
                        fills=int(dl.n_fills), fill_gb=dl.n_fills * store.blob / 1e9,
                        miss_rate_per_epoch=[float(1.0 - tr[ep == e, 3].mean()) for e in range(int(ep.max()) + 1)])

        res = dict(workload=cfg.name, layers=cfg.L, tokens_per_step=cfg.T, steps_timed=steps, steps_warmup=warm,
                   weight_sets=store.P)
        res.update(run(False))
        if cfg.epoch:
            res["epochs"] = epochs()
        res["device_control"] = bench_device(torch, cfg, store, Wrs, warm, steps, lambda st, l: xs[st][l], b)
        if cfg.act == "bf16":
            # the pages' adaptive misses: the share rate_fill / (rate_fill + rate_cpu) of misses is filled,
            # the rest runs on the host CPU from the pool (rates measured here)
            res["cpu_split"] = run(True)
        return res
    finally:
        store.close()


def profile_mxfp4(args, torch, L, gen):
    """A short run of the MXFP4 kernels for hardware-counter profiles, with every input made on the host CPU:
    no GPU work runs in the process but the library's kernels (the packer included) and the copies of their
    inputs. 16 distinct experts are generated and each packed into 16 of the 256 slots of a layer (the
    kernels' traffic and timing depend on the weights' values only through their statistics). Runs the
    4096-token MXFP4 prefill layer 3 times, one 16384-token Zipf(1.5) layer twice (groups of up to ~16k rows)
    and 48 decode FFN calls (14 experts, 48 rows: 8 tokens, top 6) on windows rotating over the 256 slots."""
    import numpy as np
    from routed_expert_layer_amd.runtime import PrefillLayer
    from workloads import CONFIGS
    dev = "cuda"
    cfg = CONFIGS["prefill_mxfp4_t4096_e256"]
    wf = L.MOE_W_MXFP4
    blob = L.moe_expert_bytes(wf, cfg.H, cfg.I)
    stride = (blob + 4095) // 4096 * 4096
    buf = torch.empty(cfg.E * stride, dtype=torch.uint8, device=dev)
    for e in range(16):
        w = {k: v.to(dev) for k, v in gen.expert_mxfp4(cfg, 0, e, "cpu").items()}
        for r in range(16):
            slot = e + 16 * r
            L.moe_pack_expert(wf, cfg.H, cfg.I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"], w["s2"],
                              buf[slot * stride:])
        section(f"profile_mxfp4: expert {e} packed")
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    out = {}
    for name, T in (("prefill_mxfp4_t4096_e256", 4096), ("prefill_db_mxfp4_t16384_l8", 16384)):
        c = CONFIGS[name]
        x = gen.tokens(c, 0, 0, "cpu").to(dev)
        Wr = gen.router_weight(c, 0, "cpu").to(dev)
        b = gen.router_bias(c, 0, 0, "cpu").to(dev)
        pl = PrefillLayer(c.H, c.I, c.E, c.k, T, stride, dev, wfmt=wf)
        reps = 3 if T == 4096 else 2
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            pl.forward(x, Wr, b, buf, s)
        torch.cuda.synchronize()
        out[name] = dict(layers=reps, ms_per_layer=(time.perf_counter() - t0) * 1e3 / reps)
        del pl
        section(f"profile_mxfp4: {name} done")
    # decode FFN: 8 tokens, 48 rows over 14 experts
    x = gen.tokens(CONFIGS["decode_mxfp4_t8_l8"], 0, 0, "cpu").to(dev)
    rows = [8, 6, 5, 4, 4, 3, 3, 3, 3, 2, 2, 2, 2, 1]
    off = np.concatenate([[0], np.cumsum(rows)])
    r = np.random.default_rng(0)
    perm_src = torch.from_numpy(np.concatenate([r.integers(0, 8, n) for n in rows]).astype(np.int32)).to(dev)
    y = torch.empty((int(off[-1]), cfg.H), dtype=torch.float32, device=dev)
    ws = torch.empty(L.moe_ffn_workspace_size(int(off[-1]), cfg.H, cfg.I, wf), dtype=torch.uint8, device=dev)
    for i in range(48):
        work = np.array([[(i * 14 + j) % cfg.E, (i * 14 + j) % cfg.E, off[j], rows[j]] for j in range(14)], np.int32)
        L.moe_ffn(x, perm_src, work, buf, stride, wf, cfg.H, cfg.I, y, ws, L.MOE_FFN_DECODE, s)
    torch.cuda.synchronize()
    out["decode_ffn_calls"] = 48
    return out


def blas_threads(torch):
    """Threads the oracle's numpy BLAS uses."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return torch.get_num_threads()


def cpu_baseline(args, torch, gen, cfg):
    """The oracle, as it stands, on a bounded sample of decode steps (host cores)."""
    import numpy as np
    import oracle
    Wr = gen.router_weight(cfg, 0, "cuda").cpu()
    b = gen.router_bias(cfg, 0, 0, "cpu")
    store = {}

    def get_expert(e):
        return store[int(e)]

    steps, spent, step = 0, 0.0, 0
    while spent < args.cpu_seconds and steps < 1024:
        x = gen.tokens(cfg, step, 0, "cuda").cpu()
        # host copies of the experts this step routes to (input preparation, untimed)
        l = oracle.router_logits(x, Wr, b)
        for e in oracle.topk_select(l, cfg.k)[0]:
            if int(e) not in store:
                store[int(e)] = tuple(t.cpu() for t in gen.expert_weights(cfg, 0, int(e), "cuda"))
        t0 = time.perf_counter()
        oracle.moe_layer(x, Wr, b, cfg.k, get_expert)
        spent += time.perf_counter() - t0
        steps += 1
        step += 1
        if len(store) > 24:
            store.clear()
    return dict(value=steps * cfg.T / spent, unit="tokens/s", cores=blas_threads(torch), kind="oracle",
                sample=f"{steps} decode steps (1 token each) of {cfg.name}, numpy fp64, "
                       f"{spent:.1f} s of oracle time; expert weights converted from bf16 inside the oracle")


def cpu_baselines_all(args, torch, gen):
    """The oracle, as it stands, per unit of the other workloads (host cores): per layer-step of the 48-layer
    stack and of the int4 8-layer decode (bounded samples), and per prefill layer of the 4096-token chunk and
    of one 16384-token layer. Routing and weight generation before each timed call are untimed input
    preparation; the oracle's own dequantisation and conversions are timed."""
    import numpy as np
    import oracle
    from workloads import CONFIGS
    out = {}

    def host_bf16(t):
        return t.cpu()

    def layer_step_rate(cfg, int4):
        Wrs, spent, n = {}, 0.0, 0
        for i in range(4096):
            st, layer = (i * 37) % cfg.steps, (i * 5) % cfg.L
            if layer not in Wrs:
                Wrs[layer] = gen.router_weight(cfg, layer, "cuda").cpu()
            x = gen.tokens(cfg, st, layer, "cuda").cpu()
            b = gen.router_bias(cfg, layer, st, "cpu")
            idx = oracle.topk_select(oracle.router_logits(x, Wrs[layer], b), cfg.k)
            raw = {}
            for e in np.unique(idx):
                if int4:
                    w = gen.expert_int4(cfg, layer, int(e), "cuda")
                    raw[int(e)] = {k_: v.cpu() for k_, v in w.items()}
                else:
                    raw[int(e)] = tuple(host_bf16(t) for t in gen.expert_weights(cfg, layer, int(e), "cuda"))

            def get_expert(e):
                if int4:
                    w = raw[int(e)]
                    return (oracle.dequant_int4(w["q1"], w["s1"], cfg.group), oracle.dequant_int4(w["q3"], w["s3"], cfg.group),
                            oracle.dequant_int4(w["q2"], w["s2"], cfg.group))
                return raw[int(e)]
            t0 = time.perf_counter()
            oracle.moe_layer(x, Wrs[layer], b, cfg.k, get_expert)
            spent += time.perf_counter() - t0
            n += 1
            if spent >= args.cpu_seconds / 2:
                break
        per = spent / n
        return dict(value=cfg.T / (per * cfg.L), unit="tokens/s", cores=blas_threads(torch), kind="oracle",
                    sample=f"{n} layer-steps of {cfg.name} ({cfg.T} tokens, {cfg.L} layers per token step), "
                           f"{spent:.1f} s of oracle time, {per * 1e3:.1f} ms per layer-step")

    def prefill_rate(cfg):
        Wr = gen.router_weight(cfg, 0, "cuda").cpu()
        b = gen.router_bias(cfg, 0, 0, "cpu")
        x = gen.tokens(cfg, 0, 0, "cuda").cpu()
        idx = oracle.topk_select(oracle.router_logits(x, Wr, b), cfg.k)
        raw = {int(e): tuple(host_bf16(t) for t in gen.expert_weights(cfg, 0, int(e), "cuda")) for e in np.unique(idx)}
        t0 = time.perf_counter()
        oracle.moe_layer(x, Wr, b, cfg.k, lambda e: raw[int(e)])
        el = time.perf_counter() - t0
        return dict(value=cfg.T / el, unit="tokens/s", cores=blas_threads(torch), kind="oracle",
                    sample=f"one whole layer of {cfg.name} ({cfg.T} tokens, {len(raw)} active experts), "
                           f"{el:.1f} s of oracle time")

    section("cpu_baseline stack48")
    out["stack48_bf16_h2048_e128"] = layer_step_rate(CONFIGS["stack48_bf16_h2048_e128"], False)
    section("cpu_baseline int4 decode")
    out["decode_int4_t8_l8"] = layer_step_rate(CONFIGS["decode_int4_t8_l8"], True)
    section("cpu_baseline prefill 4096")
    out["prefill_bf16_t4096_e256"] = prefill_rate(CONFIGS["prefill_bf16_t4096_e256"])
    section("cpu_baseline prefill 16384")
    out["prefill_db_bf16_t16384_l8"] = prefill_rate(CONFIGS["prefill_db_bf16_t16384_l8"])
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=896)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", default="decode_bf16_h4096_e256")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the int4 8-layer and 48-layer decode sections")
    ap.add_argument("--no-variants", action="store_true",
                    help="one-layer decode without its CPU-split and device-controlled variants (counter runs)")
    ap.add_argument("--no-mxfp4", action="store_true", help="skip the MXFP4 prefill and decode sections")
    ap.add_argument("--no-stack", action="store_true", help="skip the 48-layer decode section")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-all", action="store_true",
                    help="time the oracle on the one-layer decode only (not per layer-step of the stack and the "
                         "int4 decode, nor per prefill layer)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (hardware-counter calibration)")
    ap.add_argument("--profile-mxfp4", action="store_true",
                    help="only a short run of the MXFP4 kernels on inputs made on the host (counter profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X and the library has no "
              "multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    from routed_expert_layer_amd import _lib as L
    from workloads import CONFIGS, gen
    cfg = CONFIGS[args.workload]
    if cfg.phase != "decode" or cfg.wfmt != "bf16" or cfg.L != 1:
        print("bench.py times the one-layer bf16 decode workloads", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.profile_mxfp4:
        print(json.dumps({"profile_mxfp4": profile_mxfp4(args, torch, L, gen)}), flush=True)
        return
    section("decode")
    res = bench_decode(args, torch, L, gen, cfg)
    ffn = res["ffn"]
    achieved = ffn["bytes"] / (ffn["ms"] * 1e-3) / 1e9 if ffn["ms"] > 0 else 0.0
    out = {
        "metric": "MoE-layer decode tokens/s (% HBM peak); prefill expert TFLOP/s (% MFMA)",
        "value": round(res["value"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens_per_step": cfg.T, "hidden": cfg.H, "experts": cfg.E,
                   "intermediate": cfg.I, "top_k": cfg.k, "cache_slots": cfg.S, "router_zipf_s": cfg.zipf_s},
        "roofline": {"kernel": "decode expert FFN: ffn1_decode_bf16 + ffn2_combine_bf16 (the resident experts' FFN of a layer-step whose six experts were all resident, enqueued behind the routing with its work list in HBM; the down projection also forms the step's weighted output)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__))),
                     "algorithmic_bytes_per_launch": round(ffn["bytes"] / max(ffn["n"], 1)),
                     "avg_launch_us": round(ffn["ms"] * 1e3 / max(ffn["n"], 1), 2), "launches": ffn["n"]},
    }

    def rnd(d):
        return {k: (round(v, 4) if isinstance(v, float) else rnd(v) if isinstance(v, dict) else v)
                for k, v in d.items()}

    out["decode"] = rnd(res["decode"])
    out["roofline_mall_flushed"] = res["roofline_mall_flushed"]
    if not args.no_prefill:
        section("prefill")
        out["prefill"] = rnd(bench_prefill(args, torch, L, gen, CONFIGS["prefill_bf16_t4096_e256"]))
        if not args.no_mxfp4:
            section("prefill_mxfp4")
            out["prefill_mxfp4"] = rnd(bench_prefill(args, torch, L, gen, CONFIGS["prefill_mxfp4_t4096_e256"]))
        section("prefill_double_buffered")
        out["prefill_double_buffered"] = rnd(bench_prefill_pipeline(args, torch, L, gen,
                                                                    CONFIGS["prefill_db_bf16_t16384_l8"]))
        if not args.no_mxfp4:
            section("prefill_double_buffered_mxfp4")
            out["prefill_double_buffered_mxfp4"] = rnd(bench_prefill_pipeline(args, torch, L, gen,
                                                                              CONFIGS["prefill_db_mxfp4_t16384_l8"]))
    if not args.no_extra:
        section("decode_int4")
        out["decode_int4"] = rnd(bench_decode_layers(args, torch, L, gen, CONFIGS["decode_int4_t8_l8"], 64, 128))
        if not args.no_mxfp4:
            section("decode_mxfp4")
            out["decode_mxfp4"] = rnd(bench_decode_layers(args, torch, L, gen, CONFIGS["decode_mxfp4_t8_l8"], 64,
                                                          128))
        if not args.no_stack:
            section("decode_stack48")
            out["decode_stack48"] = rnd(bench_decode_layers(args, torch, L, gen, CONFIGS["stack48_bf16_h2048_e128"],
                                                            32, 64))
    if not args.no_cpu_baseline:
        section("cpu_baseline")
        cb = cpu_baseline(args, torch, gen, cfg)
        cb["value"] = round(cb["value"], 4)
        out["cpu_baseline"] = cb
        if not args.no_cpu_all:
            out["cpu_baseline_other_workloads"] = rnd(cpu_baselines_all(args, torch, gen))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
