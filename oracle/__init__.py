"""CPU oracle for the routed expert layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy (fp64) statement of what the layer
computes, plus an explicit simulator of the shared LRU expert cache. Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it. The product path (the HIP library and its Python binding) never
imports, calls or links anything in this package, and nothing in this package
imports the product path.
"""
from .moe import (  # noqa: F401
    router_logits, topk_select, topk_flags, topk_weights, permute, swiglu_expert,
    expert_outputs, combine, dequant_int4, moe_layer, e2m1_value, E2M1, e8m0_value, dequant_mxfp4,
)
from .lru import SharedLRU, TraceRec  # noqa: F401
