"""ctypes binding of libmoe.so: one Python function per C entry point, same names.

Only argument marshalling happens here (tensor -> pointer, sizes, stream
handles, status codes -> exceptions); every step of the layer runs in the HIP
library. If the library is missing this module raises on import -- there is no
fallback implementation.
"""
import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ECAPACITY, MOE_EHIP, MOE_ENOMEM, MOE_ESTATE = 0, -1, -2, -3, -4, -5
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_W_F32, MOE_W_BF16, MOE_W_INT4, MOE_W_MXFP4 = 0, 1, 2, 3
MOE_FFN_AUTO, MOE_FFN_DECODE, MOE_FFN_PREFILL = 0, 1, 2

# Every symbol include/moe.h declares.
SYMBOLS = [
    "moe_last_error", "moe_abi_version", "moe_route_workspace_size", "moe_route", "moe_expert_bytes",
    "moe_pack_expert", "moe_pool_alloc", "moe_pool_free", "moe_cache_create", "moe_cache_destroy", "cache_resolve",
    "moe_cache_trace", "moe_cache_clear_trace", "moe_cache_invalidate", "moe_cache_slot_of", "moe_cache_stats",
    "cache_fill_async", "moe_ffn_workspace_size", "moe_ffn", "moe_combine", "moe_pipe_create", "moe_pipe_destroy",
    "moe_pipe_begin_layer", "moe_pipe_end_layer", "moe_pipe_copy_ms", "moe_clock_record", "moe_decoder_create", "moe_decoder_destroy",
    "moe_decoder_step", "moe_decoder_profile", "moe_decoder_ffn_stats", "moe_decoder_fills",
    "moe_cpu_ffn", "moe_cpu_threads", "moe_cache_set_split", "moe_decoder_cpu_runs",
    "moe_device_decoder_create", "moe_device_decoder_destroy", "moe_device_decoder_step", "moe_device_decoder_stats",
    "moe_device_decoder_trace", "moe_device_decoder_clear_trace", "moe_device_decoder_slot_of",
    "moe_graph_begin", "moe_graph_end", "moe_graph_launch", "moe_graph_destroy",
    "moe_cache_resize", "moe_cache_capacity", "moe_decoder_resize", "moe_device_decoder_resize",
    "moe_ffn_grouped", "moe_prefill_layer", "moe_route_noalloc",
]


class DecoderBuffers(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("perm_src", ctypes.c_void_p),
                ("perm_pos", ctypes.c_void_p), ("y_perm", ctypes.c_void_p), ("route_ws", ctypes.c_void_p),
                ("route_ws_bytes", ctypes.c_size_t), ("ffn_ws", ctypes.c_void_p), ("ffn_ws_bytes", ctypes.c_size_t)]


class MoEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (run routed_expert_layer_amd/build.py); there is no fallback path")

_lib = ctypes.CDLL(LIB_PATH)
P = ctypes.c_void_p
I32 = ctypes.c_int
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
PI = ctypes.POINTER(ctypes.c_int)
PI64 = ctypes.POINTER(ctypes.c_int64)


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("moe_last_error", ctypes.c_char_p)
_sig("moe_abi_version", I32)
_sig("moe_route_workspace_size", SZ, I32, I32, I32, I32)
_sig("moe_route", I32, P, I32, P, P, I32, I32, I32, I32, P, P, P, P, P, P, P, P, SZ, P)
_sig("moe_route_noalloc", I32, P, I32, P, P, I32, I32, I32, I32, P, P, P, P, P, P, P, P)
_sig("moe_expert_bytes", SZ, I32, I32, I32)
_sig("moe_pack_expert", I32, I32, I32, I32, P, P, P, P, P, P, P, P)
_sig("moe_pool_alloc", P, SZ, PI)
_sig("moe_pool_free", I32, P)
_sig("moe_cache_create", P, I32, I32, I32, PI)
_sig("moe_cache_destroy", I32, P)
_sig("cache_resolve", I32, P, I32, I32, P, I32, P, P, P, P, PI, PI)
_sig("moe_cache_trace", I32, P, P, I64, PI64)
_sig("moe_cache_clear_trace", I32, P)
_sig("moe_cache_invalidate", I32, P, I32)
_sig("moe_cache_slot_of", I32, P, I32, PI)
_sig("moe_cache_stats", I32, P, PI64, PI64)
_sig("cache_fill_async", I32, P, P, I32, P, SZ, SZ, P, SZ, P, P)  # layer_pool: array of L addresses
_sig("moe_ffn_workspace_size", SZ, I32, I32, I32, I32)
_sig("moe_ffn", I32, P, I32, P, P, I32, P, SZ, I32, I32, I32, P, P, SZ, I32, P)
_sig("moe_ffn_grouped", I32, P, I32, P, P, P, P, I32, I32, I32, P, SZ, I32, I32, I32, P, P, SZ, P)
_sig("moe_combine", I32, P, P, P, I32, I32, I32, P, I32, P)
_sig("moe_pipe_create", P, P, SZ, I32, PI)
_sig("moe_pipe_destroy", I32, P)
_sig("moe_pipe_begin_layer", I32, P, I32, P, ctypes.POINTER(ctypes.c_void_p))
_sig("moe_pipe_end_layer", I32, P, I32, P)
_sig("moe_pipe_copy_ms", I32, P, I32, ctypes.POINTER(ctypes.c_float))
_sig("moe_clock_record", I32, P)
_sig("moe_decoder_create", P, P, I32, I32, I32, I32, I32, I32, I32, P, SZ, P, SZ, ctypes.POINTER(DecoderBuffers), PI)
_sig("moe_decoder_destroy", I32, P)
_sig("moe_decoder_step", I32, P, I32, I32, P, I32, P, P, P, I32, P, PI)
_sig("moe_decoder_profile", I32, P, I32)
_sig("moe_cpu_ffn", I32, P, I32, I32, I32, P, I32, P, I32)
_sig("moe_cpu_threads", I32)
_sig("moe_cache_set_split", I32, P, I32, I32)
_sig("moe_decoder_cpu_runs", I32, P, ctypes.POINTER(ctypes.c_int64))
_sig("moe_decoder_ffn_stats", I32, P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), PI64)
_sig("moe_decoder_fills", I32, P, PI64)
_sig("moe_device_decoder_create", P, I32, I32, I32, I32, I32, I32, I32, I32, I32, P, SZ, P, SZ,
     ctypes.POINTER(DecoderBuffers), I64, PI)
_sig("moe_device_decoder_destroy", I32, P)
_sig("moe_device_decoder_step", I32, P, I32, P, I32, P, P, P, I32, P)
_sig("moe_device_decoder_stats", I32, P, PI64, PI64, PI64)
_sig("moe_device_decoder_trace", I32, P, P, I64, PI64)
_sig("moe_device_decoder_clear_trace", I32, P)
_sig("moe_device_decoder_slot_of", I32, P, I32, PI)
_sig("moe_graph_begin", I32, P)
_sig("moe_graph_end", P, P, PI)
_sig("moe_graph_launch", I32, P, P)
_sig("moe_graph_destroy", I32, P)
_sig("moe_cache_resize", I32, P, I32, P, I32, PI)
_sig("moe_cache_capacity", I32, P)
_sig("moe_decoder_resize", I32, P, I32, P, P)
_sig("moe_prefill_layer", I32, P, I32, P, P, I32, I32, I32, I32, I32, I32, P, SZ, ctypes.POINTER(DecoderBuffers), P,
     I32, P)
_sig("moe_device_decoder_resize", I32, P, I32, P, P)


def _check(code, what=""):
    if code != MOE_OK:
        raise MoEError(code, (what + ": " if what else "") + _lib.moe_last_error().decode())
    return code


def _ptr(t):
    """Address of a contiguous torch tensor or numpy array, an int address (taken as given) or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("the library takes C-contiguous arrays")
        return t.ctypes.data
    if not t.is_contiguous():
        raise ValueError("the library takes contiguous tensors")
    return t.data_ptr()


def _dptr(t):
    """Address of GPU memory: a contiguous GPU tensor, an int address (taken as given) or None. A host tensor
    or array here would be read by a kernel as a device address, so it is refused."""
    if t is not None and not isinstance(t, int) and (isinstance(t, np.ndarray) or not t.is_cuda):
        raise ValueError("the library takes a GPU tensor for this argument")
    return _ptr(t)


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return MOE_DT_F32
    if t.dtype == torch.bfloat16:
        return MOE_DT_BF16
    raise ValueError(f"unsupported activation dtype {t.dtype}")


def moe_last_error():
    return _lib.moe_last_error().decode()


def moe_abi_version():
    return _lib.moe_abi_version()


# ---------------------------------------------------------------------------
def moe_route_workspace_size(T, H, E, k):
    return _lib.moe_route_workspace_size(T, H, E, k)


def moe_route(x, Wr, bias, k, topk_idx, topk_w, logits, counts, offsets, perm_src, perm_pos, workspace, stream=None):
    T, H = x.shape
    E = Wr.shape[1]
    _check(_lib.moe_route(_dptr(x), _dtype_code(x), _dptr(Wr), _dptr(bias), T, H, E, k, _dptr(topk_idx),
                          _dptr(topk_w), _dptr(logits), _dptr(counts), _dptr(offsets), _dptr(perm_src),
                          _dptr(perm_pos), _dptr(workspace), _nbytes(workspace), _stream(stream)), "moe_route")


def moe_route_noalloc(x, Wr, bias, k, topk_idx, topk_w, logits, counts, offsets, perm_src, perm_pos, stream=None):
    """moe_route with the library's own per-GPU scratch instead of a workspace argument."""
    T, H = x.shape
    E = Wr.shape[1]
    _check(_lib.moe_route_noalloc(_dptr(x), _dtype_code(x), _dptr(Wr), _dptr(bias), T, H, E, k, _dptr(topk_idx),
                                  _dptr(topk_w), _dptr(logits), _dptr(counts), _dptr(offsets), _dptr(perm_src),
                                  _dptr(perm_pos), _stream(stream)), "moe_route_noalloc")


# ---------------------------------------------------------------------------
def moe_expert_bytes(wfmt, H, I):
    return _lib.moe_expert_bytes(wfmt, H, I)


def moe_pack_expert(wfmt, H, I, W1, W3, W2, s1, s3, s2, blob, stream=None):
    _check(_lib.moe_pack_expert(wfmt, H, I, _dptr(W1), _dptr(W3), _dptr(W2), _dptr(s1), _dptr(s3), _dptr(s2), _dptr(blob),
                                _stream(stream)), "moe_pack_expert")


def moe_pool_alloc(nbytes):
    st = ctypes.c_int(0)
    p = _lib.moe_pool_alloc(nbytes, ctypes.byref(st))
    if not p:
        raise MoEError(st.value, _lib.moe_last_error().decode())
    return p


def moe_pool_free(addr):
    _check(_lib.moe_pool_free(addr), "moe_pool_free")


# ---------------------------------------------------------------------------
class MoeCache:
    """Owner of a moe_cache_t handle."""

    def __init__(self, L, E, S):
        st = ctypes.c_int(0)
        self.h = _lib.moe_cache_create(L, E, S, ctypes.byref(st))
        if not self.h:
            raise MoEError(st.value, _lib.moe_last_error().decode())
        self.L, self.E, self.S = L, E, S

    def close(self):
        if self.h and _lib is not None:  # module globals may be gone at interpreter exit
            _lib.moe_cache_destroy(self.h)
            self.h = None

    __del__ = close


def moe_cache_create(L, E, S):
    return MoeCache(L, E, S)


def moe_cache_destroy(cache):
    cache.close()


def cache_resolve(cache, step, layer, experts):
    """Returns (work_e, work_slot, work_wave, misses [n_miss, 4] = key, slot, victim, wave; n_waves)."""
    ex = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    n = len(ex)
    we = np.empty(max(n, 1), np.int32)
    ws = np.empty(max(n, 1), np.int32)
    ww = np.empty(max(n, 1), np.int32)
    ms = np.empty((max(n, 1), 4), np.int32)
    nm, nw = ctypes.c_int(0), ctypes.c_int(0)
    _check(_lib.cache_resolve(cache.h, step, layer, ex.ctypes.data, n, we.ctypes.data, ws.ctypes.data,
                              ww.ctypes.data, ms.ctypes.data, ctypes.byref(nm), ctypes.byref(nw)), "cache_resolve")
    return we[:n], ws[:n], ww[:n], ms[:nm.value], nw.value


def moe_cache_trace(cache):
    """All trace records as an int32 array [n, 7] = step, layer, key, hit, slot, victim, wave."""
    n = ctypes.c_int64(0)
    _check(_lib.moe_cache_trace(cache.h, None, 0, ctypes.byref(n)), "moe_cache_trace")
    out = np.empty((max(n.value, 1), 7), np.int32)
    _check(_lib.moe_cache_trace(cache.h, out.ctypes.data, n.value, ctypes.byref(n)), "moe_cache_trace")
    return out[:n.value]


def moe_cache_clear_trace(cache):
    _check(_lib.moe_cache_clear_trace(cache.h), "moe_cache_clear_trace")


def moe_cache_invalidate(cache, key):
    _check(_lib.moe_cache_invalidate(cache.h, key), "moe_cache_invalidate")


def moe_cache_slot_of(cache, key):
    s = ctypes.c_int(0)
    _check(_lib.moe_cache_slot_of(cache.h, key, ctypes.byref(s)), "moe_cache_slot_of")
    return s.value


def moe_cache_stats(cache):
    h, m = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.moe_cache_stats(cache.h, ctypes.byref(h), ctypes.byref(m)), "moe_cache_stats")
    return h.value, m.value


def layer_table(addrs):
    """uint64 array of per-layer host addresses (the `const void* const*` the ABI takes)."""
    return np.ascontiguousarray(np.asarray(addrs, dtype=np.uint64))


def cache_fill_async(cache, misses, layer_pool, blob_stride, blob_bytes, slot_base, slot_stride, fill_stream=None,
                     compute_stream=None):
    """layer_pool: per-layer base addresses of the pool (see layer_table)."""
    ms = np.ascontiguousarray(np.asarray(misses, dtype=np.int32).reshape(-1, 4))
    lp = layer_table(layer_pool)
    _check(_lib.cache_fill_async(cache.h, ms.ctypes.data if len(ms) else None, len(ms), lp.ctypes.data, blob_stride,
                                 blob_bytes, _dptr(slot_base), slot_stride, _stream(fill_stream),
                                 _stream(compute_stream)), "cache_fill_async")


# ---------------------------------------------------------------------------
def moe_ffn_workspace_size(rows_total, H, I, wfmt):
    return _lib.moe_ffn_workspace_size(rows_total, H, I, wfmt)


def moe_ffn(x, perm_src, work, slot_base, slot_stride, wfmt, H, I, y_perm, workspace, mode=MOE_FFN_AUTO,
            stream=None):
    """work: int32 array [n, 4] of (expert, slot, row_begin, rows)."""
    w = np.ascontiguousarray(np.asarray(work, dtype=np.int32).reshape(-1, 4))
    _check(_lib.moe_ffn(_dptr(x), _dtype_code(x), _dptr(perm_src), w.ctypes.data if len(w) else None, len(w),
                        _dptr(slot_base), slot_stride, wfmt, H, I, _dptr(y_perm), _dptr(workspace),
                        _nbytes(workspace), mode, _stream(stream)), "moe_ffn")


def moe_ffn_grouped(x, perm_src, counts, offsets, slot_of, n_slots, rows_max, slot_base, slot_stride, wfmt, H, I,
                    y_perm, workspace, stream=None):
    """counts [E], offsets [E+1], slot_of [E] or None: device int32 tensors (the work list stays on the GPU)."""
    E = counts.shape[0]
    _check(_lib.moe_ffn_grouped(_dptr(x), _dtype_code(x), _dptr(perm_src), _dptr(counts), _dptr(offsets),
                                _dptr(slot_of), E, n_slots, rows_max, _dptr(slot_base), slot_stride, wfmt, H, I,
                                _dptr(y_perm), _dptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_ffn_grouped")


def moe_combine(y_perm, perm_pos, topk_w, out, stream=None):
    T, k = perm_pos.shape
    H = y_perm.shape[1]
    _check(_lib.moe_combine(_dptr(y_perm), _dptr(perm_pos), _dptr(topk_w), T, k, H, _dptr(out), _dtype_code(out),
                            _stream(stream)), "moe_combine")


# ---------------------------------------------------------------------------
class MoePipe:
    def __init__(self, layer_src, layer_bytes):
        st = ctypes.c_int(0)
        lp = layer_table(layer_src)
        self.h = _lib.moe_pipe_create(lp.ctypes.data, layer_bytes, len(lp), ctypes.byref(st))
        if not self.h:
            raise MoEError(st.value, _lib.moe_last_error().decode())

    def close(self):
        if self.h and _lib is not None:  # module globals may be gone at interpreter exit
            _lib.moe_pipe_destroy(self.h)
            self.h = None

    __del__ = close


def moe_pipe_create(layer_src, layer_bytes):
    return MoePipe(layer_src, layer_bytes)


def moe_pipe_destroy(pipe):
    pipe.close()


def moe_pipe_begin_layer(pipe, layer, stream=None):
    buf = ctypes.c_void_p(0)
    _check(_lib.moe_pipe_begin_layer(pipe.h, layer, _stream(stream), ctypes.byref(buf)), "moe_pipe_begin_layer")
    return buf.value


def moe_pipe_end_layer(pipe, layer, stream=None):
    _check(_lib.moe_pipe_end_layer(pipe.h, layer, _stream(stream)), "moe_pipe_end_layer")


def moe_pipe_copy_ms(pipe, layer):
    ms = ctypes.c_float(0)
    _check(_lib.moe_pipe_copy_ms(pipe.h, layer, ctypes.byref(ms)), "moe_pipe_copy_ms")
    return ms.value


def moe_clock_record(sums):
    """sums: a device tensor of two int64 (zeroed by the caller), or None to turn the record off."""
    _check(_lib.moe_clock_record(_dptr(sums)), "moe_clock_record")


# ---------------------------------------------------------------------------
def _decoder_buffers(bufs):
    """DecoderBuffers from a dict of GPU tensors (names as the struct's fields)."""
    b = DecoderBuffers()
    for name in ("topk_idx", "topk_w", "logits", "counts", "offsets", "perm_src", "perm_pos", "y_perm"):
        setattr(b, name, _dptr(bufs.get(name)))
    b.route_ws, b.route_ws_bytes = _dptr(bufs["route_ws"]), _nbytes(bufs["route_ws"])
    b.ffn_ws, b.ffn_ws_bytes = _dptr(bufs["ffn_ws"]), _nbytes(bufs["ffn_ws"])
    return b


class MoeDecoder:
    """Owner of a moe_decoder_t; `bufs` maps DecoderBuffers field names to torch tensors (kept alive here)."""

    def __init__(self, cache, T_max, H, I, E, k, dtype, wfmt, layer_pool, blob_stride, slot_base, slot_stride, bufs):
        self.keep = bufs
        b = _decoder_buffers(bufs)
        st = ctypes.c_int(0)
        lp = layer_table(layer_pool)
        self.h = _lib.moe_decoder_create(cache.h, T_max, H, I, E, k, dtype, wfmt, lp.ctypes.data, blob_stride,
                                         _dptr(slot_base), slot_stride, ctypes.byref(b), ctypes.byref(st))
        if not self.h:
            raise MoEError(st.value, _lib.moe_last_error().decode())
        self.cache = cache

    def close(self):
        if self.h and _lib is not None:  # module globals may be gone at interpreter exit
            _lib.moe_decoder_destroy(self.h)
            self.h = None

    __del__ = close


def moe_decoder_create(*a, **kw):
    return MoeDecoder(*a, **kw)


def moe_decoder_destroy(dec):
    dec.close()


def moe_decoder_step(dec, step, layer, x, Wr, bias, out, stream=None):
    nm = ctypes.c_int(0)
    _check(_lib.moe_decoder_step(dec.h, step, layer, _dptr(x), x.shape[0], _dptr(Wr), _dptr(bias), _dptr(out),
                                 _dtype_code(out), _stream(stream), ctypes.byref(nm)), "moe_decoder_step")
    return nm.value


def moe_decoder_profile(dec, every):
    """every: bracket every every-th FFN call with HIP events (True = 1, False/0 = off)."""
    _check(_lib.moe_decoder_profile(dec.h, int(every)), "moe_decoder_profile")


def moe_decoder_ffn_stats(dec):
    b, m, n = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_int64(0)
    _check(_lib.moe_decoder_ffn_stats(dec.h, ctypes.byref(b), ctypes.byref(m), ctypes.byref(n)),
           "moe_decoder_ffn_stats")
    return b.value, m.value, n.value


def moe_prefill_layer(x, Wr, bias, k, I, wfmt, layer_base, blob_stride, bufs, out, stream=None):
    """bufs: a DecoderBuffers (see decoder_buffers) whose tensors the caller keeps alive."""
    T, H = x.shape
    E = Wr.shape[1]
    _check(_lib.moe_prefill_layer(_dptr(x), _dtype_code(x), _dptr(Wr), _dptr(bias), T, H, E, k, I, wfmt,
                                  _dptr(layer_base), blob_stride, ctypes.byref(bufs), _dptr(out), _dtype_code(out),
                                  _stream(stream)), "moe_prefill_layer")


def decoder_buffers(bufs):
    """The DecoderBuffers struct for a dict of GPU tensors (names as its fields)."""
    return _decoder_buffers(bufs)


def moe_decoder_fills(dec):
    n = ctypes.c_int64(0)
    _check(_lib.moe_decoder_fills(dec.h, ctypes.byref(n)), "moe_decoder_fills")
    return n.value


# ---------------------------------------------------------------------------
def moe_cpu_ffn(blob_addr, wfmt, H, I, x, y, threads=0):
    """Host expert FFN: blob_addr (int host address), x uint16/bf16 numpy [rows, H], y float32 numpy [rows, H]."""
    x = np.ascontiguousarray(x)
    assert y.flags["C_CONTIGUOUS"] and y.dtype == np.float32 and x.dtype.itemsize == 2
    _check(_lib.moe_cpu_ffn(blob_addr, wfmt, H, I, x.ctypes.data, x.shape[0], y.ctypes.data, threads), "moe_cpu_ffn")


def moe_cpu_threads():
    return _lib.moe_cpu_threads()


def moe_cache_set_split(cache, rate_gpu, rate_cpu):
    """Share of misses filled = rate_gpu / (rate_gpu + rate_cpu); the rest run on the CPU (rate_cpu = 0: all filled)."""
    _check(_lib.moe_cache_set_split(cache.h, int(rate_gpu), int(rate_cpu)), "moe_cache_set_split")


def moe_decoder_cpu_runs(dec):
    n = ctypes.c_int64(0)
    _check(_lib.moe_decoder_cpu_runs(dec.h, ctypes.byref(n)), "moe_decoder_cpu_runs")
    return n.value


# ---------------------------------------------------------------------------
class MoeDeviceDecoder:
    """Owner of a moe_device_decoder_t; `bufs` as for MoeDecoder (kept alive here)."""

    def __init__(self, L, E, S, T_max, H, I, k, dtype, wfmt, layer_pool, blob_stride, slot_base, slot_stride, bufs,
                 trace_capacity=0):
        self.keep = bufs
        b = _decoder_buffers(bufs)
        st = ctypes.c_int(0)
        lp = layer_table(layer_pool)
        self.h = _lib.moe_device_decoder_create(L, E, S, T_max, H, I, k, dtype, wfmt, lp.ctypes.data, blob_stride,
                                                _dptr(slot_base), slot_stride, ctypes.byref(b), int(trace_capacity),
                                                ctypes.byref(st))
        if not self.h:
            raise MoEError(st.value, _lib.moe_last_error().decode())

    def close(self):
        if self.h and _lib is not None:
            _lib.moe_device_decoder_destroy(self.h)
            self.h = None

    __del__ = close


def moe_device_decoder_create(*a, **kw):
    return MoeDeviceDecoder(*a, **kw)


def moe_device_decoder_destroy(dec):
    dec.close()


def moe_device_decoder_step(dec, layer, x, Wr, bias, out, stream=None):
    _check(_lib.moe_device_decoder_step(dec.h, layer, _dptr(x), x.shape[0], _dptr(Wr), _dptr(bias), _dptr(out),
                                        _dtype_code(out), _stream(stream)), "moe_device_decoder_step")


def moe_device_decoder_stats(dec):
    h, m, r = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.moe_device_decoder_stats(dec.h, ctypes.byref(h), ctypes.byref(m), ctypes.byref(r)),
           "moe_device_decoder_stats")
    return h.value, m.value, r.value


def moe_device_decoder_trace(dec, max_records):
    """int32 [n, 7] (seq, layer, key, hit, slot, victim, wave) and the number of accesses traced."""
    out = np.zeros((max(int(max_records), 1), 7), np.int32)
    n = ctypes.c_int64(0)
    _check(_lib.moe_device_decoder_trace(dec.h, out.ctypes.data, int(max_records), ctypes.byref(n)),
           "moe_device_decoder_trace")
    return out[:min(n.value, int(max_records))], n.value


def moe_device_decoder_clear_trace(dec):
    _check(_lib.moe_device_decoder_clear_trace(dec.h), "moe_device_decoder_clear_trace")


def moe_device_decoder_slot_of(dec, key):
    s = ctypes.c_int(0)
    _check(_lib.moe_device_decoder_slot_of(dec.h, key, ctypes.byref(s)), "moe_device_decoder_slot_of")
    return s.value


class MoeGraph:
    def __init__(self, h):
        self.h = h

    def close(self):
        if self.h and _lib is not None:
            _lib.moe_graph_destroy(self.h)
            self.h = None

    __del__ = close


def moe_graph_begin(stream):
    _check(_lib.moe_graph_begin(_stream(stream)), "moe_graph_begin")


def moe_graph_end(stream):
    st = ctypes.c_int(0)
    h = _lib.moe_graph_end(_stream(stream), ctypes.byref(st))
    if not h:
        raise MoEError(st.value, _lib.moe_last_error().decode())
    return MoeGraph(h)


def moe_graph_launch(graph, stream=None):
    _check(_lib.moe_graph_launch(graph.h, _stream(stream)), "moe_graph_launch")


def moe_graph_destroy(graph):
    graph.close()


# ---------------------------------------------------------------------------
def moe_cache_resize(cache, S_new):
    """Resize the host cache policy; returns int32 [n, 3] moves (key, old slot, new slot)."""
    cap = max(moe_cache_capacity(cache), 1)
    out = np.zeros((cap, 3), np.int32)
    n = ctypes.c_int(0)
    _check(_lib.moe_cache_resize(cache.h, int(S_new), out.ctypes.data, cap, ctypes.byref(n)), "moe_cache_resize")
    return out[:n.value]


def moe_cache_capacity(cache):
    return _lib.moe_cache_capacity(cache.h)


def moe_decoder_resize(dec, S_new, slot_base=None, stream=None):
    _check(_lib.moe_decoder_resize(dec.h, int(S_new), _dptr(slot_base), _stream(stream)), "moe_decoder_resize")


def moe_device_decoder_resize(dec, S_new, slot_base=None, stream=None):
    _check(_lib.moe_device_decoder_resize(dec.h, int(S_new), _dptr(slot_base), _stream(stream)),
           "moe_device_decoder_resize")
