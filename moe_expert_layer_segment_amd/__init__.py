"""MI355X (gfx950) MoE expert layer with per-request LoRA deltas.

The compute runs in hand-written HIP kernels behind a C ABI
(``include/moe_lora.h``); :mod:`.binding` is a thin ctypes layer over it and
:mod:`.workloads` generates seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    compute_moe_lora_info,
    moe_lora_align,
    moe_lora_align_capacity_rows,
    moe_lora_align_workspace_bytes,
    moe_lora_dense_forward,
    moe_lora_dense_workspace_bytes,
    moe_lora_forward,
    moe_lora_forward_workspace_bytes,
    moe_lora_info,
    moe_lora_route,
    run_dense,
    run_layer,
)
