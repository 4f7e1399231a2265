"""Chunked SGMV (segmented gather GEMM) LoRA for AMD Instinct MI355X (gfx950).

The work is done by ``libsgg_lora.so`` (C ABI in ``include/sgg_lora.h``): a
host planner and hand-written HIP kernels.  This package only marshals
arguments to it; importing it fails if the library has not been built
(``python segmented_gather_gemm_amd/build.py``).
"""

from ._lib import SggError, calls, lib
from .backend import ChunkedSgmvLoRA
from .binding import (
    LoRABatchInfo,
    default_workspace,
    lora_a_embedding,
    lora_expand,
    lora_moe_add,
    lora_moe_plan,
    lora_moe_route,
    lora_plan_device,
    lora_plan_lm_head,
    lora_plan_max_segments,
    lora_plan_segments,
    lora_qkv,
    lora_qkv_noalloc,
    lora_set_option,
    lora_shrink,
)

lib()  # load now: a missing library is an import error, never a silent fallback
calls()

__all__ = [
    "ChunkedSgmvLoRA", "LoRABatchInfo", "SggError", "default_workspace", "lora_a_embedding",
    "lora_expand", "lora_moe_add", "lora_moe_plan", "lora_moe_route", "lora_plan_device", "lora_plan_lm_head",
    "lora_plan_max_segments", "lora_plan_segments", "lora_qkv", "lora_qkv_noalloc",
    "lora_set_option", "lora_shrink",
]
