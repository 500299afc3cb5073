"""moe_route_noalloc (the routing call that allocates nothing: its scratch is a
device array the library holds per GPU) against moe_route with a caller
workspace: every output bit for bit, on two calls in a row, the second with a
smaller batch, through the C ABI. Also: a batch whose scratch exceeds the
array's size is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu
dev = "cuda"


def _outputs(T, E, k):
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(topk_idx=torch.full((T, k), -7, **i32), topk_w=torch.full((T, k), -7.0, device=dev),
                logits=torch.full((T, E), -7.0, device=dev), counts=torch.full((E,), -7, **i32),
                offsets=torch.full((E + 1,), -7, **i32), perm_src=torch.full((max(T * k, 1),), -7, **i32),
                perm_pos=torch.full((T, k), -7, **i32))


def _call(L, fn, x, Wr, b, k, o, ws=None):
    T, H = x.shape
    E = Wr.shape[1]
    args = [x.data_ptr(), L.MOE_DT_BF16 if x.dtype == torch.bfloat16 else L.MOE_DT_F32, Wr.data_ptr(),
            b.data_ptr(), T, H, E, k, o["topk_idx"].data_ptr(), o["topk_w"].data_ptr(), o["logits"].data_ptr(),
            o["counts"].data_ptr(), o["offsets"].data_ptr(), o["perm_src"].data_ptr(), o["perm_pos"].data_ptr()]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    args.append(torch.cuda.current_stream().cuda_stream)
    rc = fn(*args)
    assert rc == L.MOE_OK, L.moe_last_error()


@pytest.mark.parametrize("base,T1,T2", [("decode_bf16_h4096_e256", 16, 1), ("prefill_bf16_t4096_e256", 16384, 300),
                                         ("tiny_f32_h256_e16", 8, 3)])
def test_route_noalloc_matches_route(base, T1, T2):
    from routed_expert_layer_amd import _lib as L
    lib = L._lib
    cfg = CONFIGS[base]
    Wr = gen.router_weight(cfg, 0, dev)
    b = gen.router_bias(cfg, 0, 3, dev)
    print(f"noalloc route: {base} T={T1} then T={T2}", flush=True)
    for call, T in enumerate((T1, T2)):
        x = gen.tokens(cfg, call, 0, dev, T=T)
        ref, got = _outputs(T, cfg.E, cfg.k), _outputs(T, cfg.E, cfg.k)
        ws = torch.empty(L.moe_route_workspace_size(T, cfg.H, cfg.E, cfg.k), dtype=torch.uint8, device=dev)
        _call(L, lib.moe_route, x, Wr, b, cfg.k, ref, ws)
        _call(L, lib.moe_route_noalloc, x, Wr, b, cfg.k, got)
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(ref[name], got[name]), f"call {call} (T={T}): {name} differs"
        assert int(got["counts"].sum()) == T * cfg.k


def test_route_noalloc_refuses_oversize():
    from routed_expert_layer_amd import _lib as L
    lib = L._lib
    T, H, E, k = 16384, 4096, 1024, 6
    need = L.moe_route_workspace_size(T, H, E, k)
    assert need > (64 << 20)
    rc = lib.moe_route_noalloc(1, L.MOE_DT_BF16, 1, None, T, H, E, k, 1, 1, None, 1, 1, 1, 1, None)
    assert rc == L.MOE_ECAPACITY and "scratch" in L.moe_last_error()
