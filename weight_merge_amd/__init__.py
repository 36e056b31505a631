"""AdaFuse token-level pre-gating and one-launch fused adapter merge on MI355X.

The compute path is libadafuse.so (HIP kernels for gfx950 behind a C ABI,
include/adafuse.h); `api` is its Python binding.  PyTorch supplies device memory
and streams only.
"""
from .api import (  # noqa: F401
    AdaError,
    AdaModel,
    ada_decode_gemv,
    ada_decode_gemv_layer,
    ada_lora_apply,
    ada_lora_batch,
    ada_lora_layer,
    ada_merge,
    ada_pregate,
    ada_switch,
    ada_unmerge,
)
