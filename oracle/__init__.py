"""CPU oracle for the MoE expert layer with per-request LoRA deltas.

Test infrastructure only: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the HIP product path.  It shares no
code with the HIP path.
"""
from .moe_lora_oracle import (  # noqa: F401
    UnderCoverError,
    align_capacity_rows,
    decode_e4m3,
    dense_lora_forward,
    dequantize_block_fp8,
    moe_lora_align,
    moe_lora_forward,
    moe_lora_forward_bruteforce,
    moe_lora_info,
    moe_lora_route,
    silu,
)
