"""Seeded random tensors for the workloads in :mod:`workloads.configs`.

Every tensor has its own seed, derived from (config, tensor name, indices), so a
test can regenerate exactly the experts or steps it needs without building the
whole pool. Generation uses torch's counter-based generator on the requested
device; the same seed on the same device and torch build gives the same
values. A test that compares the HIP path with the oracle generates once and
hands the same tensors to both sides.

Nothing here computes any part of the layer. The int4 quantiser below only
turns generated weights into the int4 input format (codes and scales); the
layer itself consumes codes and scales as given.
"""
import hashlib
import math

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def seed_for(*key) -> int:
    """A 63-bit seed from an arbitrary tuple key (stable across runs)."""
    h = hashlib.blake2b(repr(key).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*key))
    return g


def normal(shape, std, key, device="cpu", dtype=torch.float32):
    """N(0, std^2) drawn in fp32, scaled, then rounded (RNE) to `dtype`."""
    g = _gen(device, *key)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def act_dtype(cfg):
    return _DT[cfg.act]


def tokens(cfg, step, layer=0, device="cpu", T=None):
    """Activations x [T, H], N(0,1), fresh per (step, layer)."""
    T = cfg.T if T is None else T
    return normal((T, cfg.H), 1.0, (cfg.name, "x", step, layer), device, act_dtype(cfg))


def router_weight(cfg, layer=0, device="cpu"):
    """Router weight Wr [H, E], std 1/sqrt(H), in the activation dtype."""
    return normal((cfg.H, cfg.E), 1.0 / math.sqrt(cfg.H), (cfg.seed_name, "Wr", layer), device, act_dtype(cfg))


def router_bias(cfg, layer=0, step=0, device="cpu"):
    """Router bias b [E] fp32: b_e = -s*ln(rank_e), rank a seeded permutation of 1..E.

    With s = 0 the bias is zero. When the config has an epoch length the
    permutation is redrawn every `epoch` steps (drifting popularity).
    """
    if cfg.zipf_s == 0.0:
        return torch.zeros(cfg.E, dtype=torch.float32, device=device)
    ep = (step // cfg.epoch) if cfg.epoch else 0
    g = _gen("cpu", cfg.seed_name, "rank", layer, ep)
    rank = torch.randperm(cfg.E, generator=g, dtype=torch.float64) + 1.0
    b = (-cfg.zipf_s * torch.log(rank)).to(torch.float32)
    return b.to(device)


def expert_weights(cfg, layer, e, device="cpu", dtype=None):
    """Canonical expert weights: W1, W3 [H, I] (std 1/sqrt(H)); W2 [I, H] (std 1/sqrt(I)).

    With cfg.pool_layers set, layer l has the weights of layer l % pool_layers.

    `dtype` defaults to the config's storage type (fp32 or bf16). For int4
    configs the bf16 weights of the same (layer, expert) are generated here and
    quantised by :func:`expert_int4`.
    """
    if dtype is None:
        dtype = torch.float32 if cfg.wfmt == "f32" else torch.bfloat16
    if cfg.pool_layers:
        layer = layer % cfg.pool_layers
    key = (cfg.seed_name, "W", layer, e)
    W1 = normal((cfg.H, cfg.I), 1.0 / math.sqrt(cfg.H), key + ("W1",), device, dtype)
    W3 = normal((cfg.H, cfg.I), 1.0 / math.sqrt(cfg.H), key + ("W3",), device, dtype)
    W2 = normal((cfg.I, cfg.H), 1.0 / math.sqrt(cfg.I), key + ("W2",), device, dtype)
    return W1, W3, W2


def quantize_int4(w, group=128):
    """Symmetric int4 codes along K (dim 0) in groups of `group`.

    s = fp16(max|w_g| / 7) (round to nearest even), q = clamp(rne(w / s), -7, 7);
    an all-zero group gets s = 0 and q = 0. Returns (q int8 [K, N], s fp16 [K/group, N]).
    """
    K, N = w.shape
    assert K % group == 0
    wf = w.to(torch.float32).reshape(K // group, group, N)
    amax = wf.abs().amax(dim=1)                       # [K/g, N]
    s = (amax / 7.0).to(torch.float16)
    sf = s.to(torch.float32)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    q = torch.round(wf / safe.unsqueeze(1))
    q = torch.where(sf.unsqueeze(1) > 0, q, torch.zeros_like(q))
    q = q.clamp_(-7, 7).to(torch.int8).reshape(K, N)
    return q, s


# FP4 (E2M1) magnitudes in code order 0..7, and the points where round-to-nearest
# moves from one to the next; ties go to the even code (mantissa bit 0).
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4(w, block=32):
    """MXFP4 codes along K (dim 0), following the OCP MX v1.0 conversion: per block
    of `block` values of a column, shared exponent X = floor(log2(max|w|)) - 2 (the
    largest FP4 exponent), scale byte X + 127 (127 for an all-zero block), codes =
    round-to-nearest-even of w / 2^X onto the FP4 grid, saturating at 6; the sign
    is kept (negative values that round to zero give code 8).
    Returns (codes uint8 [K, N] in 0..15, scales uint8 [K/block, N])."""
    K, N = w.shape
    assert K % block == 0
    wf = w.to(torch.float32).reshape(K // block, block, N)
    amax = wf.abs().amax(dim=1)                                   # [K/b, N]
    _, ex = torch.frexp(amax)                                      # amax = m * 2^ex, m in [0.5, 1)
    shared = torch.where(amax > 0, ex - 3, torch.zeros_like(ex)).clamp(-127, 127)
    v = torch.ldexp(wf, -shared.unsqueeze(1).to(torch.float32))    # exact: power-of-two scaling
    a = v.abs()
    # round to nearest, ties to even code: the boundaries below include their tie on the even side
    code = torch.zeros_like(a, dtype=torch.int32)
    code = torch.where(a > 0.25, 1, code)
    code = torch.where(a >= 0.75, 2, code)
    code = torch.where(a > 1.25, 3, code)
    code = torch.where(a >= 1.75, 4, code)
    code = torch.where(a > 2.5, 5, code)
    code = torch.where(a >= 3.5, 6, code)
    code = torch.where(a > 5.0, 7, code)
    code = code + torch.where(v < 0, 8, 0)
    return code.to(torch.uint8).reshape(K, N), (shared + 127).to(torch.uint8)


def expert_mxfp4(cfg, layer, e, device="cpu"):
    """MXFP4 expert: dict of codes c1, c3 [H, I], c2 [I, H] (uint8, 0..15) and E8M0 scales
    s1, s3 [H/32, I], s2 [I/32, H] (uint8), from the bf16 weights of the same (layer, expert)."""
    W1, W3, W2 = expert_weights(cfg, layer, e, device, torch.bfloat16)
    c1, s1 = quantize_mxfp4(W1)
    c3, s3 = quantize_mxfp4(W3)
    c2, s2 = quantize_mxfp4(W2)
    return dict(c1=c1, s1=s1, c3=c3, s3=s3, c2=c2, s2=s2)


def expert_int4(cfg, layer, e, device="cpu"):
    """int4 expert: dict of codes q1, q3 [H, I], q2 [I, H] and fp16 scales s1, s3 [H/g, I], s2 [I/g, H]."""
    W1, W3, W2 = expert_weights(cfg, layer, e, device, torch.bfloat16)
    q1, s1 = quantize_int4(W1, cfg.group)
    q3, s3 = quantize_int4(W3, cfg.group)
    q2, s2 = quantize_int4(W2, cfg.group)
    return dict(q1=q1, s1=s1, q3=q3, s3=s3, q2=q2, s2=s2)
