"""The host expert kernel (CPU execution of a missing expert) against the oracle.

Runs the library's native CPU code; no GPU involved."""
import numpy as np
import pytest
import torch

import oracle
from tests.blob_layout import bf16_bits, bf16_blob, int4_blob, mxfp4_blob
from tests.parity import check_close
from workloads import gen
import dataclasses

from workloads.configs import CONFIGS


@pytest.fixture(scope="module")
def L():
    from routed_expert_layer_amd import _lib
    return _lib


@pytest.mark.parametrize("H,I,rows", [(256, 128, 1), (256, 128, 4), (512, 384, 3), (512, 384, 8), (1024, 256, 5),
                                      (256, 128, 0)])
def test_cpu_ffn_matches_oracle(L, H, I, rows):
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name=f"cpu{H}x{I}", H=H, I=I)
    W1, W3, W2 = gen.expert_weights(cfg, 0, 3)
    blob = bf16_blob(W1, W3, W2)
    assert blob.nbytes == L.moe_expert_bytes(L.MOE_W_BF16, H, I)
    x = gen.normal((rows, H), 1.0, ("cpu-x", H, I, rows), dtype=torch.bfloat16)
    y = np.full((rows, H), np.nan, np.float32)
    L.moe_cpu_ffn(blob.ctypes.data, L.MOE_W_BF16, H, I, bf16_bits(x), y)
    if rows == 0:
        return
    ref = oracle.swiglu_expert(x.float().numpy(), W1.float().numpy(), W3.float().numpy(), W2.float().numpy())
    check_close(y, ref, f"cpu ffn H{H} I{I} rows{rows}")


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("H,I,rows", [(256, 128, 1), (512, 384, 3), (512, 384, 8), (1024, 256, 6), (256, 128, 0)])
def test_cpu_ffn_quantized_matches_oracle(L, fmt, H, I, rows):
    """int4 (codes 1 + n/16 in bf16, block sums 16 t - 24 u) and MXFP4 (E2M1 values, scales on the partial
    sums) on the host, against the oracle on the exactly dequantised weights."""
    base = "decode_int4_t8_l8" if fmt == "int4" else "decode_mxfp4_t8_l8"
    cfg = dataclasses.replace(CONFIGS[base], name=f"cpu{fmt}{H}x{I}", H=H, I=I, weights_of=None, pool_layers=None)
    if fmt == "int4":
        w = gen.expert_int4(cfg, 0, 5)
        parts = [w[k].numpy() for k in ("q1", "q3", "q2", "s1", "s3", "s2")]
        blob = int4_blob(*parts)
        W = [oracle.dequant_int4(w[q], w[s_]) for q, s_ in (("q1", "s1"), ("q3", "s3"), ("q2", "s2"))]
        wf = L.MOE_W_INT4
    else:
        w = gen.expert_mxfp4(cfg, 0, 5)
        blob = mxfp4_blob(*(w[k].numpy() for k in ("c1", "c3", "c2", "s1", "s3", "s2")))
        W = [oracle.dequant_mxfp4(w[c], w[s_]) for c, s_ in (("c1", "s1"), ("c3", "s3"), ("c2", "s2"))]
        wf = L.MOE_W_MXFP4
    assert blob.nbytes == L.moe_expert_bytes(wf, H, I)
    x = gen.normal((rows, H), 1.0, ("cpu-q4x", fmt, H, I, rows), dtype=torch.bfloat16)
    y = np.full((rows, H), np.nan, np.float32)
    L.moe_cpu_ffn(blob.ctypes.data, wf, H, I, bf16_bits(x), y)
    if rows == 0:
        return
    ref = oracle.swiglu_expert(x.float().numpy(), *W)
    check_close(y, ref, f"cpu ffn {fmt} H{H} I{I} rows{rows}")


def test_cpu_ffn_thread_counts_agree(L):
    H, I, rows = 512, 256, 6
    cfg = dataclasses.replace(CONFIGS["decode_bf16_h4096_e256"], name="cputh", H=H, I=I)
    W1, W3, W2 = gen.expert_weights(cfg, 0, 1)
    blob = bf16_blob(W1, W3, W2)
    x = bf16_bits(gen.normal((rows, H), 1.0, ("cpu-th",), dtype=torch.bfloat16))
    outs = []
    for th in (1, 2, L.moe_cpu_threads()):
        y = np.empty((rows, H), np.float32)
        L.moe_cpu_ffn(blob.ctypes.data, L.MOE_W_BF16, H, I, x, y, th)
        outs.append(y)
    # every output element is one thread's fixed-order sum: identical for any split
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_cpu_ffn_rejects(L):
    y = np.empty((1, 64), np.float32)
    x = np.zeros((1, 64), np.uint16)
    blob = np.zeros(3 * 64 * 64, np.uint16)
    for wfmt, H, I in [(L.MOE_W_F32, 64, 64), (L.MOE_W_INT4, 64, 128), (L.MOE_W_MXFP4, 128, 96),
                       (L.MOE_W_BF16, 48, 64)]:
        with pytest.raises(L.MoEError) as ei:
            L.moe_cpu_ffn(blob.ctypes.data, wfmt, H, I, x, y)
        assert ei.value.code == L.MOE_EINVAL
