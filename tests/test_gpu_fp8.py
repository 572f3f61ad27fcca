"""GPU parity of the layer with fp8 expert weights (OCP e4m3 codes, 128 x 128
block scales, power-of-two or general fp32; x, LoRA pools and y in bf16) against the oracle, which decodes
the codes from the format's definition and dequantizes in float64.

The bar is the bf16 layer bar: the kernels convert each code exactly and round
code * scale to bf16 before the matrix cores, an error of at most half a bf16
ulp per weight, of the same order as the bf16 rounding of the activations."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_layer_close, gate_up_tail_split, gpu_inputs, oracle_forward, run, say, to_np
from moe_expert_layer_segment_amd import workloads

pytestmark = pytest.mark.gpu

SMALL = [
    # name, E, k, H, I, L, ranks, seg_lens, weight_indices, R
    ("fp8_tiles", 8, 2, 256, 384, 4, [0, 8, 16, 16], [40, 1, 77, 3, 90, 29], [2, 0, 3, 2, -1, 1], 16),
    ("fp8_ragged_down_cols", 6, 3, 384, 256, 3, [32, 12, 5], [33, 64, 7], [0, 1, 2], 32),
    ("fp8_rank64_long_k", 16, 4, 1024, 512, 5, [64, 0, 8, 64, 33], [100, 50, 150, 10], [0, 4, 3, -1], 64),
    ("fp8_one_token", 4, 1, 128, 128, 2, [8, 8], [1], [1], 8),
    # >= 64 pairs per expert: the 128-deep K tiles of prefill-sized batches
    ("fp8_deep_k", 2, 2, 512, 384, 3, [16, 0, 32], [70, 50, 80], [0, 1, 2], 32),
]


def _y32(inp, **kw):
    y32 = run(inp, out_dtype=torch.float32, **kw)
    y16 = run(inp, **kw)
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 y is not the rounded fp32 y"
    return to_np(y32)


@pytest.mark.parametrize("scales", ["fp8", "fp8_f32scale"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_small_full(case, scales):
    # power-of-two block scales take the scaled conversion instruction, other
    # fp32 scales the exact multiply; both round code * scale to bf16
    name, E, k, H, I, L, ranks, lens, wi, R = case
    say(f"forward fp8 small {name} ({scales})")
    spec = workloads.LayerSpec(name, E, k, H, I, L, ranks, lens, wi, seed=19, pool_rank=R,
                               weights=scales)
    inp = gpu_inputs(spec)
    assert inp["w_gate_up"].dtype == torch.uint8
    sc = inp["w_gate_up_scale"]
    assert bool(torch.all(torch.exp2(torch.round(torch.log2(sc))) == sc)) == (scales == "fp8")
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", f"{name} {scales}")


def test_fp8_base_only():
    spec = workloads.LayerSpec("fp8_base", 8, 2, 256, 256, 2, [16, 16], [20, 30], [0, 1],
                               seed=20, pool_rank=16, weights="fp8")
    say("forward fp8 without LoRA")
    inp = gpu_inputs(spec, with_lora=False)
    got = to_np(run(inp, with_lora=False, out_dtype=torch.float32))
    assert_layer_close(got, oracle_forward(inp, with_lora=False), "bf16", "fp8 base")


@pytest.mark.parametrize("E,lens", [(4, [30, 1, 25, 8]), (2, [70, 50, 80])],
                         ids=["decode_tiles", "deep_k_tiles"])
def test_fp8_down_k_split(E, lens):
    spec = workloads.LayerSpec("fp8_down_k_split", E, 2, 128, 8192, 2, [16, 8], lens,
                               [0, -1, 1, 0][:len(lens)], seed=28, pool_rank=16, weights="fp8")
    say(f"forward fp8 with the down GEMM's K split (I = 8192, E = {E})")
    inp = gpu_inputs(spec)
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", "fp8 down K split")


@pytest.mark.parametrize("scales", ["fp8", "fp8_f32scale"])
@pytest.mark.parametrize("E,H,I,lens", [(64, 4096, 256, [20, 30, 14]), (4, 8192, 768, [100, 100, 100])],
                         ids=["decode_tiles", "deep_k_tiles"])
def test_fp8_gate_up_tail_split(E, H, I, lens, scales):
    """Few work items for the grid: the fp8 gate_up GEMM hands its last tiles out
    as K pieces, each taking the block scales from its own first K tile, and a
    second kernel adds them.  Every token against the oracle."""
    spec = workloads.LayerSpec("fp8_tail_split", E, 2, H, I, 3, [16, 0, 32], lens, [0, 2, -1], seed=2,
                               pool_rank=32, router="uniform_bias", weights=scales)
    split = gate_up_tail_split(spec)
    say(f"forward fp8 tail split E={E} H={H} ({scales}): (xcd, full rounds, tail tiles, pieces) {split}")
    assert split, "the shape no longer exercises the tail split"
    inp = gpu_inputs(spec)
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", f"fp8 tail split E={E} {scales}")


@pytest.mark.parametrize("name,n_sample", [("c1_fp8", 40), ("c4p_fp8", 12), ("c3_fp8", 0),
                                           ("c4d_fp8", 0)])
def test_fp8_full_size(name, n_sample):
    """Prefill batches on a strided token sample; the decode batches (64 and 128
    tokens) on every token (n_sample 0)."""
    spec = workloads.config(name)
    say(f"forward full-size {name}: T={spec.num_tokens}")
    inp = gpu_inputs(spec)
    got = to_np(run(inp, out_dtype=torch.float32))
    assert np.all(np.isfinite(got))
    T = spec.num_tokens
    if n_sample:
        sample = np.unique(np.concatenate([np.linspace(0, T - 1, n_sample).astype(np.int64),
                                           [0, T - 1]]))
        ref = oracle_forward(inp, tokens=sample)
        assert_layer_close(got[sample], ref, "bf16", f"{name} ({len(sample)} sampled tokens)")
    else:
        ref = oracle_forward(inp)
        assert_layer_close(got, ref, "bf16", f"{name} (all {T} tokens)")
    del inp
    torch.cuda.empty_cache()
