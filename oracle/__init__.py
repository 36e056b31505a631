"""CPU oracle (fp64, NumPy) for the AdaFuse pre-gating and fused-merge path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.
"""
from .adafuse import (  # noqa: F401
    adapter_delta,
    gate_weights,
    gemv,
    merge,
    pregate,
    router_logits,
    routed_lora_forward,
    select_topk,
    switch,
    unmerge,
)
