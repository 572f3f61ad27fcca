"""Helpers shared by the GPU parity tests: host views of device inputs for the
oracle, and the parity metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from moe_expert_layer_segment_amd import binding, workloads

POOLS = ("a_gate", "a_up", "b_gate", "b_up", "a_down", "b_down")

# acceptance bars for the layer output against the float64 oracle (bf16:
# relative L2 and max abs; fp32: relative L2)
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 5e-2
F32_REL_L2 = 1e-4


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class HostView:
    """Lazy float64 host copy of a device tensor, one index at a time (the
    oracle reads only the experts / slots the sampled tokens touch)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, idx):
        key = idx if isinstance(idx, tuple) else (idx,)
        key = tuple(int(i) for i in key)
        return self.t[key].float().cpu().numpy().astype(np.float64)


class Fp8HostView:
    """fp8 e4m3 expert weights seen by the oracle: each expert's codes and
    block scales copied to the host and dequantized by the oracle on access
    (the last expert is kept, since the oracle reads one expert at a time)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        self.codes, self.scales = codes, scales
        self._e, self._w = None, None

    def __getitem__(self, idx):
        key = idx if isinstance(idx, tuple) else (idx,)
        e = int(key[0])
        if self._e != e:
            self._w = oracle.dequantize_block_fp8(self.codes[e].cpu().numpy(),
                                                  self.scales[e].cpu().numpy())
            self._e = e
        return self._w[tuple(int(i) for i in key[1:])] if len(key) > 1 else self._w


def weight_views(inp: dict):
    """(w_gate_up, w_down) host views for the oracle, dequantizing fp8 weights."""
    if "w_gate_up_scale" in inp:
        return (Fp8HostView(inp["w_gate_up"], inp["w_gate_up_scale"]),
                Fp8HostView(inp["w_down"], inp["w_down_scale"]))
    return HostView(inp["w_gate_up"]), HostView(inp["w_down"])


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.int32, torch.int64):
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


def oracle_forward(inp: dict, tokens=None, with_lora=True):
    """Oracle y (float64) for the device inputs ``inp`` of workloads.generate."""
    m = inp["meta"]
    T = inp["x"].shape[0]
    en, mp = oracle.moe_lora_info(T, m["seg_indptr"], m["weight_indices"], m["lora_ranks"],
                                  m["max_seg_len"])
    w_gu, w_d = weight_views(inp)
    kw = dict(x=to_np(inp["x"]) if tokens is None else HostView(inp["x"]),
              topk_ids=m["topk_ids"], topk_weights=m["topk_weights"],
              w_gate_up=w_gu, w_down=w_d,
              lora_ranks=m["lora_ranks"], scaling=m["scaling"],
              token_lora_mapping=mp, adapter_enabled=en, tokens=tokens)
    if with_lora and "a_gate" in inp:
        for n in POOLS:
            kw[n] = HostView(inp[n])
    return oracle.moe_lora_forward(**kw)


def metrics(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    return rel, mx


def assert_layer_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel, mx = metrics(got, ref)
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    if dtype == "f32":
        assert rel <= F32_REL_L2, (what, rel)
    else:
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, (what, rel, mx)


def gpu_inputs(spec, canary=True, with_lora=True):
    return workloads.generate(spec, device="cuda", canary=canary, with_lora=with_lora)


def run(inp, block_m=16, with_lora=True, out_dtype=None):
    y = binding.run_layer(inp, block_m=block_m, with_lora=with_lora, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def gate_up_tail_split(spec, block_m=16):
    """Which XCD ranges of the general gate_up GEMM split their tail tiles into
    K pieces, recomputed from the library's rule: the host's grid (from its
    bound on work items), the device's item count (from the oracle's align),
    per-XCD tile ranges of ceil(tiles / 8), and for a range of n_x tiles on
    wx = grid / 8 workgroups a tail r = n_x % wx with 0 < 4 r <= wx split into
    S = min(wx / r, K tiles / 2) pieces (S >= 2; only when K has >= 64 K tiles).
    Returns (xcd, full rounds, tail tiles, pieces) of each splitting range."""
    bf = spec.dtype == "bf16"
    rpi, BN, per_cu, BK = (128, 256, 1, 64) if bf else (64, 64, 2, 32)
    T = int(sum(spec.seg_lens))
    P = T * spec.top_k
    if spec.weights.startswith("fp8"):   # 128-deep K tiles from 64 pairs per expert on
        BK = 128 if P >= 64 * spec.num_experts else 64
    ids, _ = workloads.route(workloads.router_logits(spec), spec.top_k)
    seg = np.concatenate([[0], np.cumsum(spec.seg_lens)]).astype(np.int32)
    en, mp = oracle.moe_lora_info(T, seg, np.array(spec.weight_indices, np.int32),
                                  np.array(spec.lora_ranks, np.int32), max(spec.seg_lens))
    al = oracle.moe_lora_align(ids.astype(np.int32), mp, en, spec.num_experts, spec.num_loras, block_m)
    cap = oracle.align_capacity_rows(P, spec.num_experts, spec.num_loras, block_m)
    max_items = -(-cap // rpi) + min(P, spec.num_experts)
    n_tiles = -(-spec.inter // (BN // 2))
    grid = min(256 * per_cu, -(-n_tiles * max_items // 8) * 8)
    eto = al["expert_tile_offsets"]
    count = min(max_items, sum(-(-int(eto[e + 1] - eto[e]) * block_m // rpi) for e in range(spec.num_experts)))
    total, wx, nk = count * n_tiles, grid // 8, spec.hidden // BK
    if nk < 64:
        return []
    per = -(-total // 8)
    out = []
    for x in range(8):
        n_x = max(0, min(total, (x + 1) * per) - x * per)
        q, r = divmod(n_x, wx)
        if 0 < r and 4 * r <= wx and min(wx // r, nk // 2) >= 2:
            out.append((x, q, r, min(wx // r, nk // 2)))
    return out
