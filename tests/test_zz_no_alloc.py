"""The allocation-free forward (moe_lora_forward_noalloc, through the C ABI)
against moe_lora_forward: bit-identical outputs on two calls in a row, the
second with a smaller problem (the static scratch keeps the first call's
contents), for bf16 and fp32 layers."""
import pytest
import torch

from gpu_helpers import gpu_inputs, say
from moe_expert_layer_segment_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _both(spec):
    inp = gpu_inputs(spec)
    T, k = inp["topk_ids"].shape
    E, L = spec.num_experts, spec.num_loras
    en, mp = binding.moe_lora_info(T, inp["seg_indptr"], inp["lora_ranks"], inp["weight_indices"])
    al = binding.moe_lora_align(inp["topk_ids"], mp, en, E, L, 16)
    pools = {n: inp[n] for n in binding._POOLS}
    args = (inp["x"], inp["topk_weights"], inp["w_gate_up"], inp["w_down"], al, k,
            inp["lora_ranks"], inp["scaling"], pools)
    need = binding.moe_lora_forward_workspace_bytes(*args)
    assert need <= binding.moe_lora_forward_noalloc_max_workspace_bytes(), need
    y_ref = binding.moe_lora_forward(*args).clone()
    y = torch.full_like(y_ref, float("nan"))
    binding.moe_lora_forward_noalloc(*args, y=y)
    torch.cuda.synchronize()
    return y, y_ref, need


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_forward_twice(dtype):
    big = workloads.config("c3") if dtype == "bf16" else workloads.LayerSpec(
        "na_f32_big", 16, 4, 512, 768, 6, [8, 16, 0, 32, 16, 8], [90, 40, 120, 33, 77],
        [0, 5, 2, -1, 3], dtype="f32", seed=31, pool_rank=32)
    small = workloads.LayerSpec("na_small", 8, 2, 256, 384, 4, [0, 8, 16, 16],
                                [40, 1, 17, 3, 9, 29], [2, 0, 3, 2, -1, 1], dtype=dtype, seed=32,
                                pool_rank=16)
    for spec in (big, small):
        y, y_ref, need = _both(spec)
        say(f"  noalloc {spec.name} ({dtype}): workspace {need / 2**20:.1f} MiB")
        assert torch.equal(y, y_ref), spec.name
