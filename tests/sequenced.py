"""A decode layer-step sequenced from the individual C-ABI calls (test helper).

The library's decode driver (moe_decoder_step) runs the whole layer-step in
one call. This helper issues the same steps one entry point at a time from
Python -- moe_route, cache_resolve, cache_fill_async per wave, moe_ffn per
wave, moe_combine -- so the tests check that the separate calls compose into
the same layer as the driver. It is test code: the product path is the
driver.
"""
import numpy as np
import torch

from routed_expert_layer_amd import _lib as L
from routed_expert_layer_amd.runtime import RouteBuffers


class SequencedDecodeLayer:
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
        self.n_fills = 0
        self.cpu_runs = 0

    def step(self, step, layer, x, Wr, bias, stream=None):
        s = stream or torch.cuda.current_stream()
        T = x.shape[0]
        rb = self.rb
        rb.route(x, Wr, bias, s)
        counts, off = rb.fetch_counts(s)
        experts = np.nonzero(counts)[0].astype(np.int32)
        we, wslot, wwave, misses, n_waves = L.cache_resolve(self.cache, step, layer, experts)
        for w in range(n_waves):
            m = misses[misses[:, 3] == w]
            if len(m):
                L.cache_fill_async(self.cache, m, self.store.layer_ptrs, self.store.stride, self.store.blob,
                                   self.slots, self.store.stride, self.fill_stream, s)
                self.n_fills += len(m)
            sel = wwave == w
            e = we[sel]
            work = np.stack([e, wslot[sel], off[e], counts[e]], axis=1).astype(np.int32)
            L.moe_ffn(x, rb.perm_src, work, self.slots, self.store.stride, self.store.wfmt, self.H, self.I,
                      self.y_perm, self.ffn_ws, L.MOE_FFN_AUTO, s)
        L.moe_combine(self.y_perm, rb.perm_pos[:T], rb.topk_w[:T], self.out[:T], s)
        return self.out[:T]

    def resize(self, n_slots, stream=None):
        """moe_cache_resize plus the blob copies it asks for (and, growing, the kept blobs into a new buffer)."""
        s = stream or torch.cuda.current_stream()
        old = self.slots
        new = None
        if n_slots > self.S:
            new = torch.empty(n_slots * self.store.stride, dtype=torch.uint8, device=old.device)
        moves = L.moe_cache_resize(self.cache, n_slots)
        st = self.store.stride
        with torch.cuda.stream(s):
            dst = old if new is None else new
            if new is not None:
                for key in range(self.store.L * self.E):
                    sl = L.moe_cache_slot_of(self.cache, key)
                    if sl >= 0 and not any(m[0] == key for m in moves):
                        dst[sl * st:(sl + 1) * st].copy_(old[sl * st:(sl + 1) * st])
            for key, a, b in moves:
                dst[b * st:(b + 1) * st].copy_(old[a * st:(a + 1) * st])
        if new is not None:
            self.keep_old = old  # read by copies on the stream
            self.slots = new
        self.S = n_slots

    def trace(self):
        return L.moe_cache_trace(self.cache)
