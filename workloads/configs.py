"""The synthetic workloads the layer is tested and measured on.

Shapes follow the published model family the pages describe (six of 256
routed experts per layer, page "FreeToken-rtx-4090", section "How the MoE
Memory Hierarchy Works") and the five workload descriptions this project was
given: a tiny fp32 layer, a one-layer bf16 decode, a 48-layer shared-cache
decode stack, a 4096-token prefill chunk, and an 8-layer prefill with
double buffering followed by an int4 decode phase on the same layers.

Reading of "N(0, 1/sqrt(fan_in))": standard deviation 1/sqrt(fan_in).
Reading of "router bias drawn Zipf(s)": b_e = -s * ln(rank_e) with rank a
seeded permutation of 1..E, which makes expert popularity Zipf-skewed.

The 8-layer bf16 pool (8 x 12.88 GB) exceeds the ~64 GiB of page-locked host
memory the test machines allow, so its layers share four weight sets (layer l
uses set l % 4); routers and biases stay distinct per layer and every layer is
still copied in full, so the transfer volume is unchanged.
"""
from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    L: int                 # layers
    T: int                 # tokens per step (decode) or per layer (prefill)
    steps: int             # decode steps (1 for prefill)
    H: int                 # hidden size
    E: int                 # routed experts per layer
    I: int                 # SwiGLU intermediate size
    k: int                 # experts per token
    act: str               # activation/router dtype: "f32" | "bf16"
    wfmt: str              # expert weight format: "f32" | "bf16" | "int4" | "mxfp4"
    zipf_s: float = 0.0    # router-bias skew (0: no bias)
    epoch: Optional[int] = None   # bias re-permuted every `epoch` steps
    S: Optional[int] = None       # cache slots (None: every expert resident)
    phase: str = "decode"  # "decode" | "prefill"
    weights_of: Optional[str] = None  # reuse another config's layer weights
    pool_layers: Optional[int] = None  # distinct weight sets; layer l uses set l % pool_layers
    group: int = 128       # int4 group size along K
    extra: dict = field(default_factory=dict)

    @property
    def seed_name(self):
        return self.weights_of or self.name


CONFIGS = {
    # tiny fp32 layer, 64-step routing trace over an 8-slot cache
    "tiny_f32_h256_e16": Config("tiny_f32_h256_e16", L=1, T=8, steps=64, H=256, E=16, I=128, k=2,
                                act="f32", wfmt="f32", zipf_s=0.0, S=8),
    # one-layer bf16 decode, batch 1, 64 of 256 experts cached
    "decode_bf16_h4096_e256": Config("decode_bf16_h4096_e256", L=1, T=1, steps=1024, H=4096, E=256, I=2048,
                                     k=6, act="bf16", wfmt="bf16", zipf_s=1.1, S=64),
    # 48-layer stack, batch 4, shared cache of 2048 of 6144 layer-expert entries
    "stack48_bf16_h2048_e128": Config("stack48_bf16_h2048_e128", L=48, T=4, steps=512, H=2048, E=128, I=768,
                                      k=8, act="bf16", wfmt="bf16", zipf_s=1.2, epoch=128, S=2048),
    # 4096-token prefill chunk, all experts resident, unbiased router
    "prefill_bf16_t4096_e256": Config("prefill_bf16_t4096_e256", L=1, T=4096, steps=1, H=4096, E=256, I=2048,
                                      k=6, act="bf16", wfmt="bf16", zipf_s=0.0, phase="prefill"),
    # the same 4096-token chunk with the same experts in MXFP4
    "prefill_mxfp4_t4096_e256": Config("prefill_mxfp4_t4096_e256", L=1, T=4096, steps=1, H=4096, E=256, I=2048,
                                       k=6, act="bf16", wfmt="mxfp4", zipf_s=0.0, phase="prefill",
                                       weights_of="prefill_bf16_t4096_e256"),
    # 8-layer prefill, 16384 tokens per layer, Zipf(1.5) routing, double-buffered layer copies
    "prefill_db_bf16_t16384_l8": Config("prefill_db_bf16_t16384_l8", L=8, T=16384, steps=1, H=4096, E=256,
                                        I=2048, k=6, act="bf16", wfmt="bf16", zipf_s=1.5, phase="prefill",
                                        pool_layers=4),
    # the same 8-layer prefill with MXFP4 experts (eight distinct weight sets: 27.4 GB of pool)
    "prefill_db_mxfp4_t16384_l8": Config("prefill_db_mxfp4_t16384_l8", L=8, T=16384, steps=1, H=4096, E=256,
                                         I=2048, k=6, act="bf16", wfmt="mxfp4", zipf_s=1.5, phase="prefill",
                                         weights_of="prefill_db_bf16_t16384_l8"),
    # MXFP4 decode on the same 8 layers (the same bf16 weights in the OCP MX FP4 format), batch 8,
    # 512-entry shared cache
    "decode_mxfp4_t8_l8": Config("decode_mxfp4_t8_l8", L=8, T=8, steps=256, H=4096, E=256, I=2048, k=6,
                                 act="bf16", wfmt="mxfp4", zipf_s=1.5, S=512,
                                 weights_of="prefill_db_bf16_t16384_l8", pool_layers=4),
    # int4 decode on the same 8 layers, batch 8, 512-entry shared cache
    "decode_int4_t8_l8": Config("decode_int4_t8_l8", L=8, T=8, steps=256, H=4096, E=256, I=2048, k=6,
                                act="bf16", wfmt="int4", zipf_s=1.5, S=512,
                                weights_of="prefill_db_bf16_t16384_l8", pool_layers=4),
}


def get_config(name: str, **overrides) -> Config:
    """Return a named config, optionally with fields overridden (for cut-down cases)."""
    import dataclasses
    c = CONFIGS[name]
    return dataclasses.replace(c, **overrides) if overrides else c
