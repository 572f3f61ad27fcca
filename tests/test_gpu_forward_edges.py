"""GPU parity of the layer on the degenerate and extreme cases of the method:
an empty batch, requests of length zero, every pair routed to one expert,
every token routed to every expert, the largest expert x slot key space
the align step supports (E * (L + 1) = 32768), a batch large enough for the
shrinks to share pool rows across row groups, and an intermediate size long
enough for the down GEMM to split K."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_layer_close, gpu_inputs, oracle_forward, run, say, to_np
from moe_expert_layer_segment_amd import workloads

pytestmark = pytest.mark.gpu


def _y32(inp, **kw):
    return to_np(run(inp, out_dtype=torch.float32, **kw))


def _force_routing(inp, ids: np.ndarray, w: np.ndarray):
    """Replace the router's choice (device tensors and the oracle's host copy)."""
    inp = dict(inp)
    inp["topk_ids"] = torch.from_numpy(ids.astype(np.int32)).cuda()
    inp["topk_weights"] = torch.from_numpy(w.astype(np.float32)).cuda()
    inp["meta"] = dict(inp["meta"], topk_ids=ids.astype(np.int32), topk_weights=w.astype(np.float32))
    return inp


def test_empty_batch():
    spec = workloads.LayerSpec("empty", 4, 2, 64, 128, 2, [8, 8], [0, 0], [0, 1], seed=21,
                               pool_rank=8)
    say("forward edge: empty batch")
    inp = gpu_inputs(spec)
    y = run(inp)
    assert tuple(y.shape) == (0, 64)
    y32 = run(inp, out_dtype=torch.float32)
    assert tuple(y32.shape) == (0, 64)


def test_zero_length_requests():
    spec = workloads.LayerSpec("zero_len", 6, 2, 128, 192, 3, [16, 0, 8],
                               [0, 37, 0, 0, 20, 0, 5], [1, 0, 2, 1, -1, 0, 2], seed=22,
                               pool_rank=16)
    say("forward edge: requests of length zero")
    inp = gpu_inputs(spec)
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", "zero-length requests")


@pytest.mark.parametrize("k", [1, 2])
def test_every_pair_on_one_expert(k):
    # 300 tokens x k pairs all on experts {3, 3+1, ..}: 300-row buckets span
    # several 128-row work items and end ragged
    T = 300
    spec = workloads.LayerSpec("one_expert", 8, k, 128, 256, 4, [16, 8, 0, 16],
                               [120, 100, 80], [0, 3, 1], seed=23, pool_rank=16)
    say(f"forward edge: every pair on one expert (k={k})")
    inp = gpu_inputs(spec)
    ids = np.tile(np.arange(3, 3 + k, dtype=np.int32), (T, 1))
    w = np.full((T, k), 1.0 / k, dtype=np.float32)
    inp = _force_routing(inp, ids, w)
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", f"one expert k={k}")


def test_top_k_equals_num_experts():
    spec = workloads.LayerSpec("all_experts", 4, 4, 128, 128, 2, [8, 16], [33, 30], [1, 0],
                               seed=24, pool_rank=16)
    say("forward edge: top_k = E")
    inp = gpu_inputs(spec)
    T = spec.num_tokens
    ids = np.tile(np.arange(4, dtype=np.int32), (T, 1))
    rng = np.random.default_rng(24)
    w = rng.random((T, 4)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    inp = _force_routing(inp, ids, w)
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", "top_k = E")


def test_largest_expert_slot_key_space():
    # E = 256, L = 127: E * (L + 1) = 32768, the align step's limit; a few
    # live slots spread over the pool, the rest rank 0
    L = 127
    ranks = [8 if l % 31 == 1 else 0 for l in range(L)]
    nreq = 12
    wi = [(7 * b) % L for b in range(nreq)]
    wi[0] = 1                      # a live slot
    wi[1] = 32                     # another live slot
    wi[2] = -1
    spec = workloads.LayerSpec("key_space", 256, 4, 64, 64, L, ranks, [5] * nreq, wi, seed=25,
                               pool_rank=8)
    say("forward edge: E * (L + 1) = 32768")
    inp = gpu_inputs(spec)
    assert_layer_close(_y32(inp), oracle_forward(inp), "bf16", "E*(L+1)=32768")


@pytest.mark.parametrize("dtype,block_m", [("bf16", 16), ("bf16", 128), ("f32", 16)])
def test_large_batch_shared_pool_shrink(dtype, block_m):
    # over 64K pairs with large (expert, slot) buckets: the shrinks share each
    # bucket's pool rows across 4 row groups; with 16-row tiles many 4-group
    # spans straddle two buckets (the groups of the other bucket read their pool
    # rows directly), and slot 1 has rank 0
    rng = np.random.default_rng(26)
    segs = [int(v) for v in rng.integers(200, 1600, size=48)]
    wi = [int(v) for v in rng.integers(-1, 3, size=48)]
    spec = workloads.LayerSpec("shared_shrink", 4, 2, 128, 192, 3, [16, 0, 12], segs, wi,
                               dtype=dtype, seed=26, pool_rank=16)
    assert spec.num_tokens * spec.top_k >= 65536
    say(f"forward edge: shared-pool shrink, {spec.num_tokens} tokens, {dtype}, block_m={block_m}")
    inp = gpu_inputs(spec)
    assert_layer_close(_y32(inp, block_m=block_m), oracle_forward(inp), dtype,
                       f"shared-pool shrink {dtype} bm={block_m}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_down_gemm_k_split(dtype):
    # a long intermediate size and few tiles: the down GEMM splits K in two
    # (two fp32 planes of z, added by the combine in order); the LoRA expand
    # is added in the first split only
    spec = workloads.LayerSpec("down_k_split", 4, 2, 128, 8192, 2, [16, 8], [30, 1, 25, 8],
                               [0, -1, 1, 0], dtype=dtype, seed=27, pool_rank=16)
    say(f"forward edge: down GEMM K split, I = 8192, {dtype}")
    inp = gpu_inputs(spec)
    assert_layer_close(_y32(inp), oracle_forward(inp), dtype, f"down K split {dtype}")
