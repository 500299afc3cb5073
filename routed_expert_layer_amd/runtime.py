"""Sequencing of the C-ABI calls into a decode layer-step and a prefill layer.

No arithmetic of the layer happens here: routing, expert FFN and combine run in
the HIP library, the cache policy in its C++ host code, and the fills as
host-to-device copies it issues. This module owns the buffers (torch device
tensors, page-locked host memory from the library) and the order of calls.

Page "FreeToken-rtx-4090": the complete expert pool lives in host memory, the
GPU holds a cache of complete layer-and-expert entries (section "How the MoE
Memory Hierarchy Works"); decode resolves each step's experts against a shared
LRU and moves only the missing ones (component table, rows "GPU memory" and
"PCIe link"); prefill streams the next layer's experts while the current layer
computes (phase table, row "Prefill").
"""
import ctypes

import time

import numpy as np
import torch

from . import _lib as L

WFMT = {"f32": L.MOE_W_F32, "bf16": L.MOE_W_BF16, "int4": L.MOE_W_INT4, "mxfp4": L.MOE_W_MXFP4}


def _align(v, a):
    return (v + a - 1) // a * a


def host_view(addr, nbytes):
    """A CPU uint8 tensor over library-owned page-locked memory (no copy)."""
    buf = (ctypes.c_uint8 * nbytes).from_address(addr)
    return torch.frombuffer(buf, dtype=torch.uint8, count=nbytes)


class ExpertStore:
    """The experts of L layers as packed blobs in page-locked host memory.

    One pinned region per physical layer; layer l reads physical layer
    l % phys_layers (phys_layers < L lets several layers share the same weights
    when the machine cannot pin a full pool). Blob of expert e of layer l is at
    layer_ptrs[l] + e * stride.
    """

    def __init__(self, n_layers, E, H, I, wfmt, phys_layers=None):
        self.L, self.E, self.H, self.I = n_layers, E, H, I
        self.P = n_layers if phys_layers is None else phys_layers
        self.wfmt = WFMT[wfmt] if isinstance(wfmt, str) else wfmt
        self.blob = L.moe_expert_bytes(self.wfmt, H, I)
        if self.blob == 0:
            raise ValueError(f"unsupported expert shape {H}x{I} for format {wfmt}")
        self.stride = _align(self.blob, 4096)
        self.layer_bytes = E * self.stride
        self.nbytes = self.P * self.layer_bytes
        self.phys, self.views = [], []
        try:
            for _ in range(self.P):
                a = L.moe_pool_alloc(self.layer_bytes)
                self.phys.append(a)
                self.views.append(host_view(a, self.layer_bytes))
        except Exception:
            self.close()
            raise
        self.layer_ptrs = L.layer_table([self.phys[l % self.P] for l in range(n_layers)])

    def pack_layer(self, layer, make_expert, device="cuda", batch=16):
        """Pack every expert of physical layer `layer` into the pool.

        make_expert(e) returns canonical device tensors: (W1, W3, W2) for fp32/bf16,
        a dict with q1, q3, q2 (int8) and s1, s3, s2 (fp16) for int4, or a dict with
        c1, c3, c2 (uint8 FP4 codes) and s1, s3, s2 (uint8 E8M0 scales) for MXFP4.
        """
        assert 0 <= layer < self.P
        stage = torch.empty(batch * self.stride, dtype=torch.uint8, device=device)
        view = self.views[layer]
        for e0 in range(0, self.E, batch):
            n = min(batch, self.E - e0)
            for j in range(n):
                w = make_expert(e0 + j)
                dst = stage[j * self.stride:]
                if self.wfmt == L.MOE_W_INT4:
                    L.moe_pack_expert(self.wfmt, self.H, self.I, w["q1"], w["q3"], w["q2"], w["s1"], w["s3"],
                                      w["s2"], dst)
                elif self.wfmt == L.MOE_W_MXFP4:
                    L.moe_pack_expert(self.wfmt, self.H, self.I, w["c1"], w["c3"], w["c2"], w["s1"], w["s3"],
                                      w["s2"], dst)
                else:
                    L.moe_pack_expert(self.wfmt, self.H, self.I, w[0], w[1], w[2], None, None, None, dst)
            off = e0 * self.stride
            view[off:off + n * self.stride].copy_(stage[:n * self.stride])
        torch.cuda.synchronize()

    def close(self):
        self.views = []
        for a in self.phys:
            L.moe_pool_free(a)
        self.phys = []


class RouteBuffers:
    """Device outputs of moe_route for up to T tokens."""

    def __init__(self, T, H, E, k, device="cuda", keep_logits=False):
        self.T, self.H, self.E, self.k = T, H, E, k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device) if keep_logits else None
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm_src = torch.empty(max(T * k, 1), **i32)
        self.perm_pos = torch.empty((T, k), **i32)
        self.ws = torch.empty(L.moe_route_workspace_size(T, H, E, k), dtype=torch.uint8, device=device)
        self.counts_host = torch.empty(E, dtype=torch.int32, pin_memory=True)
        self.offsets_host = torch.empty(E + 1, dtype=torch.int32, pin_memory=True)

    def route(self, x, Wr, bias, stream=None):
        T = x.shape[0]
        assert T <= self.T
        L.moe_route(x, Wr, bias, self.k, self.topk_idx[:T], self.topk_w[:T],
                    None if self.logits is None else self.logits[:T], self.counts, self.offsets, self.perm_src,
                    self.perm_pos[:T], self.ws, stream)

    def fetch_counts(self, stream=None):
        """Device-to-host copies of the per-expert counts and offsets the routing kernels wrote; waits for them."""
        s = stream or torch.cuda.current_stream()
        with torch.cuda.stream(s):
            self.counts_host.copy_(self.counts, non_blocking=True)
            self.offsets_host.copy_(self.offsets, non_blocking=True)
        s.synchronize()
        return self.counts_host.numpy().astype(np.int64), self.offsets_host.numpy().astype(np.int64)

    def buffer_dict(self, y_perm, ffn_ws):
        """The device buffers of a layer call (DecoderBuffers field names)."""
        return dict(topk_idx=self.topk_idx, topk_w=self.topk_w, logits=self.logits, counts=self.counts,
                    offsets=self.offsets, perm_src=self.perm_src, perm_pos=self.perm_pos, y_perm=y_perm,
                    route_ws=self.ws, ffn_ws=ffn_ws)


class DecodeLayer:
    """Decode path: route -> host LRU -> fills -> grouped FFN -> combine, for one cache, one call per layer-step
    through the library's decode driver (moe_decoder_step)."""

    def __init__(self, store, n_slots, T, k, act, device="cuda", keep_logits=False):
        self.store, self.S, self.k = store, n_slots, k
        self.H, self.I, self.E = store.H, store.I, store.E
        self.act = act
        self.rb = RouteBuffers(T, self.H, self.E, k, device, keep_logits)
        self.cache = L.MoeCache(store.L, store.E, n_slots)
        self.slots = torch.empty(n_slots * store.stride, dtype=torch.uint8, device=device)
        rows = T * k
        self.y_perm = torch.empty((max(rows, 1), self.H), dtype=torch.float32, device=device)
        self.ffn_ws = torch.empty(L.moe_ffn_workspace_size(rows, self.H, self.I, store.wfmt), dtype=torch.uint8,
                                  device=device)
        self.out = torch.empty((T, self.H), dtype=torch.float32, device=device)
        self.fill_stream = torch.cuda.Stream(device=device)
        self.dec = L.MoeDecoder(self.cache, T, self.H, self.I, self.E, k,
                                L.MOE_DT_BF16 if act == "bf16" else L.MOE_DT_F32, store.wfmt, store.layer_ptrs,
                                store.stride, self.slots, store.stride, self.rb.buffer_dict(self.y_perm, self.ffn_ws))

    @property
    def n_fills(self):
        return L.moe_decoder_fills(self.dec)

    @property
    def cpu_runs(self):
        """Misses executed on the CPU so far."""
        return L.moe_decoder_cpu_runs(self.dec)

    def resize(self, n_slots, stream=None):
        """Change the cache to n_slots slots between layer-steps (the most recently used entries stay); a larger
        cache gets a new slot buffer, into which the kept blobs are copied on the stream."""
        s = stream or torch.cuda.current_stream()
        new = None
        if n_slots > self.S:
            new = torch.empty(n_slots * self.store.stride, dtype=torch.uint8, device=self.slots.device)
        L.moe_decoder_resize(self.dec, n_slots, new, s)
        if new is not None:
            self.keep_old = self.slots  # read by copies on the stream
            self.slots = new
        self.S = n_slots

    def set_split(self, rate_gpu, rate_cpu):
        """Divide misses between GPU fills and CPU execution in the ratio of the rates (e.g. MB/s of pinned
        fills and of the host expert kernel, see measure_rates); rate_cpu = 0 fills every miss."""
        L.moe_cache_set_split(self.cache, rate_gpu, rate_cpu)

    def measure_rates(self, layer=0, n=4, rows=None):
        """(fill MB/s, CPU expert MB/s) on this machine: n pinned blobs of `layer` copied to a scratch device
        buffer on the fill stream, and the host expert kernel on the same blobs with `rows` token rows."""
        store = self.store
        n = max(1, min(n, store.E - 1))
        tmp = torch.empty(n * store.stride, dtype=torch.uint8, device=self.slots.device)
        misses = [[layer * store.E + e, e, -1, 0] for e in range(n)]
        fs = self.fill_stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(fs)
        L.cache_fill_async(self.cache, misses, store.layer_ptrs, store.stride, store.blob, tmp, store.stride, fs, fs)
        e1.record(fs)
        torch.cuda.synchronize()
        fill_mbs = n * store.blob / (e0.elapsed_time(e1) * 1e-3) / 1e6
        del tmp
        rows = rows or self.rb.T
        x = torch.randn(rows, self.H).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        y = np.empty((rows, self.H), np.float32)
        base = int(store.layer_ptrs[layer])
        # warm the thread pool on an expert outside the timed set, so that no timed blob is in the host's caches
        L.moe_cpu_ffn(base + (store.E - 1) * store.stride, store.wfmt, self.H, self.I, x, y)
        t0 = time.perf_counter()
        for e in range(n):
            L.moe_cpu_ffn(base + e * store.stride, store.wfmt, self.H, self.I, x, y)
        cpu_mbs = n * store.blob / (time.perf_counter() - t0) / 1e6
        return fill_mbs, cpu_mbs

    def step(self, step, layer, x, Wr, bias, stream=None):
        """One layer-step (blocks until the step's counts reach the host; the rest is enqueued on the stream)."""
        s = stream or torch.cuda.current_stream()
        T = x.shape[0]
        L.moe_decoder_step(self.dec, step, layer, x, Wr, bias, self.out[:T], s)
        return self.out[:T]

    def trace(self):
        return L.moe_cache_trace(self.cache)


class DeviceDecodeLayer:
    """Decode path with the cache control in GPU memory (moe_device_decoder_*): routing, the resolve kernel, the
    fill kernel, the FFN over the device work list and the combine are enqueued with no host synchronisation,
    so a sequence of layer-steps can be captured once (capture) and replayed (replay) on static buffers."""

    def __init__(self, store, n_slots, T, k, act, device="cuda", keep_logits=False, trace_capacity=0):
        self.store, self.S, self.k, self.T = store, n_slots, k, T
        self.H, self.I, self.E = store.H, store.I, store.E
        self.act = act
        self.rb = RouteBuffers(T, self.H, self.E, k, device, keep_logits)
        self.slots = torch.empty(n_slots * store.stride, dtype=torch.uint8, device=device)
        rows = T * k
        self.y_perm = torch.empty((max(rows, 1), self.H), dtype=torch.float32, device=device)
        self.ffn_ws = torch.empty(L.moe_ffn_workspace_size(rows, self.H, self.I, store.wfmt), dtype=torch.uint8,
                                  device=device)
        self.out = torch.empty((T, self.H), dtype=torch.float32, device=device)
        rb = self.rb
        bufs = dict(topk_idx=rb.topk_idx, topk_w=rb.topk_w, logits=rb.logits, counts=rb.counts, offsets=rb.offsets,
                    perm_src=rb.perm_src, perm_pos=rb.perm_pos, y_perm=self.y_perm, route_ws=rb.ws,
                    ffn_ws=self.ffn_ws)
        self.dec = L.MoeDeviceDecoder(store.L, self.E, n_slots, T, self.H, self.I, k,
                                      L.MOE_DT_BF16 if act == "bf16" else L.MOE_DT_F32, store.wfmt,
                                      store.layer_ptrs, store.stride, self.slots, store.stride, bufs, trace_capacity)

    def resize(self, n_slots, stream=None):
        """Change the cache to n_slots slots at a safe point (waits for the stream); a larger cache gets a new
        slot buffer. Graphs captured earlier must be captured again."""
        s = stream or torch.cuda.current_stream()
        new = None
        if n_slots > self.S:
            new = torch.empty(n_slots * self.store.stride, dtype=torch.uint8, device=self.slots.device)
        L.moe_device_decoder_resize(self.dec, n_slots, new, s)
        if new is not None:
            self.slots = new  # the copies have finished: the call waits for them
        self.S = n_slots

    def step(self, layer, x, Wr, bias, stream=None, out=None):
        """Enqueue one layer-step; returns the output tensor (valid once the stream reaches it)."""
        s = stream or torch.cuda.current_stream()
        o = self.out[:x.shape[0]] if out is None else out
        L.moe_device_decoder_step(self.dec, layer, x, Wr, bias, o, s)
        return o

    @staticmethod
    def capture(enqueue, stream):
        """Record the work `enqueue()` puts on `stream` (a torch.cuda.Stream) into a graph; nothing runs."""
        L.moe_graph_begin(stream)
        try:
            enqueue()
        finally:
            g = L.moe_graph_end(stream)
        return g

    @staticmethod
    def replay(graph, stream):
        L.moe_graph_launch(graph, stream)

    def stats(self):
        """(hits, misses, resolve calls) so far; synchronises the device."""
        torch.cuda.synchronize()
        return L.moe_device_decoder_stats(self.dec)

    @property
    def n_fills(self):
        return self.stats()[1]

    def trace(self, max_records):
        torch.cuda.synchronize()
        return L.moe_device_decoder_trace(self.dec, max_records)


class PrefillLayer:
    """Prefill path over a layer whose experts are all resident (blob of expert e at base + e*stride): one
    moe_prefill_layer call enqueues routing, the grouped GEMM over the work list planned on the GPU and the
    combine; nothing waits for the GPU."""

    def __init__(self, H, I, E, k, T, stride, device="cuda", keep_logits=False, wfmt=L.MOE_W_BF16):
        self.H, self.I, self.E, self.k, self.stride, self.wfmt = H, I, E, k, stride, wfmt
        self.rb = RouteBuffers(T, H, E, k, device, keep_logits)
        rows = T * k
        self.y_perm = torch.empty((max(rows, 1), H), dtype=torch.float32, device=device)
        self.ffn_ws = torch.empty(L.moe_ffn_workspace_size(rows, H, I, wfmt), dtype=torch.uint8, device=device)
        self.out = torch.empty((T, H), dtype=torch.float32, device=device)
        self.bufs = L.decoder_buffers(self.rb.buffer_dict(self.y_perm, self.ffn_ws))

    def forward(self, x, Wr, bias, layer_base, stream=None, timer=None):
        """Enqueue the layer on the stream; returns the output tensor (valid once the stream reaches it).
        With `timer`, the same three steps are enqueued as separate calls (moe_route, moe_ffn_grouped,
        moe_combine) and timer.begin/end(stream, expert FLOPs) bracket the grouped FFN."""
        s = stream or torch.cuda.current_stream()
        T = x.shape[0]
        rb = self.rb
        if timer is None:
            L.moe_prefill_layer(x, Wr, bias, self.k, self.I, self.wfmt, layer_base, self.stride, self.bufs,
                                self.out[:T], s)
            return self.out[:T]
        rb.route(x, Wr, bias, s)
        timer.begin(s)
        self.ffn(x, layer_base, T, s)
        timer.end(s, 6.0 * self.H * self.I * T * self.k)  # expert FLOPs of the T*k routed pairs
        L.moe_combine(self.y_perm, rb.perm_pos[:T], rb.topk_w[:T], self.out[:T], s)
        return self.out[:T]

    def ffn(self, x, layer_base, T=None, stream=None):
        """The grouped expert FFN alone on the routing the buffers hold."""
        T = x.shape[0] if T is None else T
        L.moe_ffn_grouped(x, self.rb.perm_src, self.rb.counts, self.rb.offsets, None, self.E, T * self.k,
                          layer_base, self.stride, self.wfmt, self.H, self.I, self.y_perm, self.ffn_ws, stream)
