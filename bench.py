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
matrix-core peak; and the CPU oracle on a bounded sample of the same decode
workload.

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
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


def measured_traffic(root):
    """HBM bytes per FFN call from the committed counter summary, if the kernel sources are unchanged since."""
    import hashlib
    path = os.path.join(root, "profiles", "decode_ffn_hbm_traffic.json")
    try:
        j = json.load(open(path))
        for rel, digest in j["sources_sha256"].items():
            if hashlib.sha256(open(os.path.join(root, rel), "rb").read()).hexdigest() != digest:
                return None
        return int(j["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def percentile(xs, p):
    xs = sorted(xs)
    if not xs:
        return 0.0
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


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
    L.moe_decoder_profile(dl.dec, True)  # HIP events around every expert-FFN call, on stream s
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
        decode=dict(step_ms_p50=percentile(lat, 50) * 1e3, step_ms_p99=percentile(lat, 99) * 1e3,
                    step_ms_max=max(lat) * 1e3, hit_rate=hit_rate, fills_timed=dl.n_fills - fills0,
                    fills_warmup=fills0, fill_gbs=fill_gbs, fill_frac_pcie=fill_gbs / PCIE_PEAK_GBS,
                    pool_gb=store.nbytes / 1e9, slots=cfg.S),
    )


def bench_prefill(args, torch, L, gen, cfg, reps=5):
    from routed_expert_layer_amd.runtime import PrefillLayer
    dev = "cuda"
    blob = L.moe_expert_bytes(L.MOE_W_BF16, cfg.H, cfg.I)
    stride = (blob + 4095) // 4096 * 4096
    buf = torch.empty(cfg.E * stride, dtype=torch.uint8, device=dev)
    for e in range(cfg.E):
        W1, W3, W2 = gen.expert_weights(cfg, 0, e, dev)
        L.moe_pack_expert(L.MOE_W_BF16, cfg.H, cfg.I, W1, W3, W2, None, None, None, buf[e * stride:])
    pl = PrefillLayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, stride, dev)
    Wr = gen.router_weight(cfg, 0, dev)
    b = gen.router_bias(cfg, 0, 0, dev)
    x = gen.tokens(cfg, 0, 0, dev)
    for _ in range(2):
        pl.forward(x, Wr, b, buf)
    timer = EventTimer(torch, reps)
    timer.enabled = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        pl.forward(x, Wr, b, buf, timer=timer)
    torch.cuda.synchronize()
    layer_ms = (time.perf_counter() - t0) * 1e3 / reps
    flops, ms, n = timer.result()
    active = int((pl.last_counts > 0).sum())
    tfs = flops / (ms * 1e-3) / 1e12
    wbytes = active * blob
    del buf
    return dict(workload=cfg.name, tokens=cfg.T, layer_ms=layer_ms, gemm_ms=ms / n, tflops=tfs,
                mfma_frac=tfs / MFMA_BF16_PEAK_TFS, weight_gbs=wbytes / (ms / n * 1e-3) / 1e9,
                hbm_frac=wbytes / (ms / n * 1e-3) / 1e9 / HBM_PEAK_GBS, active_experts=active,
                group_min=int(pl.last_counts[pl.last_counts > 0].min()), group_max=int(pl.last_counts.max()))


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
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = torch.get_num_threads()
    return dict(value=steps * cfg.T / spent, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{steps} decode steps (1 token each) of {cfg.name}, numpy fp64, "
                       f"{spent:.1f} s of oracle time; expert weights converted from bf16 inside the oracle")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=896)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", default="decode_bf16_h4096_e256")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (hardware-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X and this build has no "
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
        "roofline": {"kernel": "decode expert FFN: ffn1_decode_bf16 + ffn2_decode_bf16 (one moe_ffn call)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__))),
                     "algorithmic_bytes_per_launch": round(ffn["bytes"] / max(ffn["n"], 1)),
                     "avg_launch_us": round(ffn["ms"] * 1e3 / max(ffn["n"], 1), 2), "launches": ffn["n"]},
        "decode": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in res["decode"].items()},
    }
    if not args.no_prefill:
        p = bench_prefill(args, torch, L, gen, CONFIGS["prefill_bf16_t4096_e256"])
        out["prefill"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in p.items()}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args, torch, gen, cfg)
        cb["value"] = round(cb["value"], 4)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
