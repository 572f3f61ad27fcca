"""One GPU's share of the layer under tensor and expert parallelism.

Tensor parallelism splits the intermediate dimension I: W_gate/W_up and the
B_g/B_u pools by their output rows, W_down and the A_d pool along I, with A_g,
A_u and B_d replicated; each rank's output is a partial y and the ranks' sum is
the layer (the down expand is linear in the split h).  Expert parallelism gives
each rank E/G experts; the dispatched (token, expert) pairs arrive as rows
routed to one local expert, and the returned rows are summed per token.

The tests run every rank of a small layer (2, 4 and 8 ranks) on this GPU and check that the ranks
add up to the oracle's layer, and run the per-rank kernel at the full shard
shapes (c1 with TP=8, c4 with EP=8) against the oracle on sampled tokens."""
import numpy as np
import pytest
import torch

from gpu_helpers import POOLS, assert_layer_close, gpu_inputs, oracle_forward, run, say, to_np
from moe_expert_layer_segment_amd import workloads

pytestmark = pytest.mark.gpu


def _tp_shard(inp, G, g, I):
    """Rank g of G: slices of the intermediate dimension (column-parallel
    gate/up and B_g/B_u, row-parallel down and A_d)."""
    Ig = I // G
    sl = slice(g * Ig, (g + 1) * Ig)
    out = dict(inp)
    wgu = inp["w_gate_up"]
    out["w_gate_up"] = torch.cat([wgu[:, sl], wgu[:, I + g * Ig:I + (g + 1) * Ig]], dim=1).contiguous()
    out["w_down"] = inp["w_down"][:, :, sl].contiguous()
    for n in ("b_gate", "b_up", "a_down"):
        out[n] = inp[n][..., sl].contiguous()
    return out


@pytest.mark.parametrize("G", [2, 4, 8])
def test_tp_ranks_sum_to_layer(G):
    spec = workloads.LayerSpec("tp", 8, 2, 256, 512, 3, [16, 8, 0], [45, 30, 21], [0, 1, 2],
                               seed=51, pool_rank=16)
    say(f"TP={G} ranks of a small layer")
    inp = gpu_inputs(spec)
    total = None
    for g in range(G):
        shard = _tp_shard(inp, G, g, spec.inter)
        y = to_np(run(shard, out_dtype=torch.float32))
        if g == 0:
            # a rank on its own against the oracle on the same slices
            assert_layer_close(y, oracle_forward(shard), "bf16", "TP rank 0")
        total = y if total is None else total + y
    assert_layer_close(total, oracle_forward(inp), "bf16", "sum of TP ranks")


@pytest.mark.parametrize("G", [2, 4, 8])
def test_ep_ranks_sum_to_layer(G):
    spec = workloads.LayerSpec("ep", 8, 2, 256, 256, 3, [16, 8, 16], [40, 27, 33], [0, 1, 2],
                               seed=52, pool_rank=16)
    say(f"EP={G} ranks of a small layer")
    inp = gpu_inputs(spec)
    m = inp["meta"]
    T, k = m["topk_ids"].shape
    E, H = spec.num_experts, spec.hidden
    Eg = E // G
    mapping = np.repeat(m["weight_indices"], np.diff(m["seg_indptr"]))
    y = np.zeros((T, H))
    for r in range(G):
        tt, jj = np.nonzero((m["topk_ids"] >= r * Eg) & (m["topk_ids"] < (r + 1) * Eg))
        if tt.size == 0:
            continue
        # the rows this rank receives: one per local pair, each its own request
        ids = (m["topk_ids"][tt, jj] - r * Eg).astype(np.int32)[:, None]
        w = m["topk_weights"][tt, jj].astype(np.float32)[:, None]
        rank = dict(inp)
        rank["x"] = inp["x"][torch.from_numpy(tt).cuda()].contiguous()
        rank["topk_ids"] = torch.from_numpy(ids).cuda()
        rank["topk_weights"] = torch.from_numpy(w).cuda()
        rank["w_gate_up"] = inp["w_gate_up"][r * Eg:(r + 1) * Eg].contiguous()
        rank["w_down"] = inp["w_down"][r * Eg:(r + 1) * Eg].contiguous()
        for n in POOLS:
            rank[n] = inp[n][:, r * Eg:(r + 1) * Eg].contiguous()
        seg = np.arange(tt.size + 1, dtype=np.int32)
        wi = mapping[tt].astype(np.int32)
        rank["seg_indptr"] = torch.from_numpy(seg).cuda()
        rank["weight_indices"] = torch.from_numpy(wi).cuda()
        rank["meta"] = dict(m, seg_indptr=seg, weight_indices=wi, topk_ids=ids, topk_weights=w,
                            max_seg_len=1)
        yr = to_np(run(rank, out_dtype=torch.float32))
        np.add.at(y, tt, yr)
    assert_layer_close(y, oracle_forward(inp), "bf16", "sum of EP ranks")


@pytest.mark.parametrize("name", workloads.SHARD_CONFIG_NAMES)
def test_shard_shapes_sampled(name):
    spec = workloads.config(name)
    say(f"shard shape {name}: T={spec.num_tokens} E={spec.num_experts} I={spec.inter}")
    inp = gpu_inputs(spec)
    got = to_np(run(inp, out_dtype=torch.float32))
    T = spec.num_tokens
    sample = np.unique(np.concatenate([np.linspace(0, T - 1, 32).astype(np.int64), [0, T - 1]]))
    ref = oracle_forward(inp, tokens=sample)
    assert_layer_close(got[sample], ref, spec.dtype, f"{name} ({len(sample)} sampled tokens)")
    del inp
    torch.cuda.empty_cache()
