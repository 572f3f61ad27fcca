"""Seeded synthetic inputs for the MoE expert layer with per-request LoRA deltas.

This module only *generates inputs*: request segments, adapter slots, router
outputs, expert weights and LoRA pools.  It holds none of the layer's own
arithmetic (no projection, activation, LoRA delta or combine), so that both the
HIP path and the CPU oracle can be fed from it without sharing any computation.
It imports nothing else from this package.

Shapes and distributions follow the workloads of the MoE-LoRA pages
(SGLang PR #14105 "LoRA on MoE expert layers", section "实现拆解": the 4-D pool
[num_loras, num_experts, rank, dim]; SGLang PR #24160, section "关键源码片段":
int32 segment / adapter metadata).  Conventions fixed here where the pages are
silent:

* ``N(m, v)`` takes ``v`` as the variance: W ~ N(0, 1/fan_in), A ~ N(0, 1/in),
  B ~ N(0, 0.01) (std 0.1).
* Pools are rank-major: A as [L, E, R, in], B stored transposed as
  [L, E, R, out].  Rows at index >= the slot rank are NaN when ``canary`` is
  set (they must never be read) and 0 otherwise.
* Router: float64 softmax over experts, top-k by descending probability with
  ties going to the lower expert id, weights renormalised over the top-k and
  stored as float32.
* Each expert weight has its own sub-seed derived from ``(seed, tensor_id,
  expert)``, and each LoRA pool slot (all experts at once) from ``(seed,
  tensor_id, slot)``, so any expert or slot can be regenerated on its own.  A
  pool is drawn with one call per slot, which keeps the number of device
  launches of a large configuration in the hundreds.
* fp8 expert weights: each expert's fp32 draw is quantized to OCP e4m3 codes
  over 128 x 128 blocks; x, pools and y stay bf16.  ``weights="fp8"`` uses
  power-of-two block scales, 2^ceil(log2(amax / 448)) (448 = the largest finite
  e4m3 value; the UE8M0 scale recipe); ``weights="fp8_f32scale"`` uses
  scale = amax / 448 exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

# tensor ids for sub-seeds
_TID_X, _TID_WGU, _TID_WD = 1, 2, 3
_TID_AG, _TID_AU, _TID_BG, _TID_BU, _TID_AD, _TID_BD = 4, 5, 6, 7, 8, 9
_TID_ROUTER, _TID_LENS, _TID_WI, _TID_RANKS, _TID_BIAS = 10, 11, 12, 13, 14


@dataclasses.dataclass
class LayerSpec:
    """One MoE-LoRA layer plus one batch of requests."""
    name: str
    num_experts: int
    top_k: int
    hidden: int
    inter: int
    num_loras: int
    lora_ranks: List[int]
    seg_lens: List[int]
    weight_indices: List[int]
    dtype: str = "bf16"          # "bf16" or "f32": x, weights, pools and y
    seed: int = 0
    router: str = "normal"       # "normal" | "zipf" | "uniform_bias"
    alpha_over_rank: float = 2.0  # scaling = alpha / r with alpha = 2r
    pool_rank: Optional[int] = None
    weights: str = "same"        # "same" (dtype), "fp8" / "fp8_f32scale": e4m3 codes + 128 x 128 block scales

    @property
    def num_tokens(self) -> int:
        return int(sum(self.seg_lens))

    @property
    def num_reqs(self) -> int:
        return len(self.seg_lens)

    @property
    def max_rank(self) -> int:
        if self.pool_rank is not None:
            return int(self.pool_rank)
        return max([int(r) for r in self.lora_ranks] + [1])

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def _subseed(*key: int) -> int:
    ss = np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key])
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(_subseed(*key))


def _lengths_with_total(rng: np.random.Generator, bs: int, total: int,
                        lo: int = 64, hi: int = 512) -> List[int]:
    """Request lengths drawn U{lo..hi}, then nudged one token at a time (a seeded
    random request, staying within [lo, hi]) until they sum to ``total``."""
    if not (bs * lo <= total <= bs * hi):
        raise ValueError("total not reachable with lengths in [lo, hi]")
    lens = rng.integers(lo, hi + 1, size=bs).astype(np.int64)
    while lens.sum() != total:
        b = int(rng.integers(0, bs))
        if lens.sum() > total and lens[b] > lo:
            lens[b] -= 1
        elif lens.sum() < total and lens[b] < hi:
            lens[b] += 1
    return [int(v) for v in lens]


def config(name: str) -> LayerSpec:
    """The six named workloads (c4 has a prefill batch and a decode batch)."""
    if name == "c0":
        # tiny fp32 layer, request structure of the pages' worked example
        return LayerSpec("c0_tiny_fp32", 8, 2, 256, 512, 4, [0, 8, 8, 16],
                         [5, 1, 7, 3, 9, 2], [2, 0, 3, 2, -1, 1],
                         dtype="f32", seed=0, router="normal", pool_rank=16)
    if name == "c1":
        seed = 1
        rng = _rng(seed, _TID_LENS)
        lens = _lengths_with_total(rng, 16, 4096)
        rng = _rng(seed, _TID_WI)
        wi = rng.integers(0, 8, size=16)
        neg = rng.choice(16, size=2, replace=False)   # 10% of 16 requests -> 2
        wi[neg] = -1
        ranks = [0] + [16] * 7
        return LayerSpec("c1_mixtral_prefill", 8, 2, 4096, 14336, 8, ranks, lens,
                         [int(v) for v in wi], seed=seed, router="normal",
                         pool_rank=16)
    if name == "c2":
        seed = 2
        lens = _lengths_with_total(_rng(seed, _TID_LENS), 32, 8192)
        ranks = _rng(seed, _TID_RANKS).choice([0, 8, 16, 32, 64], size=16)
        wi = _rng(seed, _TID_WI).integers(0, 16, size=32)
        return LayerSpec("c2_finegrained_prefill", 128, 8, 2048, 768, 16,
                         [int(r) for r in ranks], lens, [int(v) for v in wi],
                         seed=seed, router="zipf",
                         pool_rank=int(max(ranks)) if max(ranks) > 0 else 8)
    if name == "c3":
        return LayerSpec("c3_decode", 128, 8, 2048, 768, 32, [32] * 32, [1] * 64,
                         [b % 32 for b in range(64)], seed=3, router="normal",
                         pool_rank=32)
    if name in ("c4p", "c4d"):
        if name == "c4p":
            lens = _lengths_with_total(_rng(4, _TID_LENS), 64, 16384)
            wi = [int(v) for v in _rng(4, _TID_WI).integers(0, 8, size=64)]
        else:
            lens = [1] * 128
            wi = [b % 8 for b in range(128)]
        return LayerSpec(f"{name}_large_expert_{'prefill' if name == 'c4p' else 'decode'}",
                         256, 8, 7168, 2048, 8, [32] * 8, lens, wi, seed=4,
                         router="uniform_bias", pool_rank=32)
    if name in ("c1_tp2", "c1_tp4", "c1_tp8"):
        # one rank of c1 under G-way tensor parallelism: I split G ways
        G = int(name[len("c1_tp"):])
        c1 = config("c1")
        return LayerSpec(f"c1_tp{G}_rank", c1.num_experts, c1.top_k, c1.hidden, c1.inter // G,
                         c1.num_loras, c1.lora_ranks, c1.seg_lens, c1.weight_indices,
                         seed=c1.seed, router=c1.router, pool_rank=c1.pool_rank)
    if name in ("c4p_ep8", "c4d_ep8"):
        # one rank of c4 under 8-way expert parallelism: 32 local experts; each
        # dispatched (token, expert) pair arrives as a row routed to one expert
        # (k = 8 pairs per token, 1/8 of them local: about one row per token)
        c4 = config(name[:3])
        lens, wi = c4.seg_lens, c4.weight_indices
        return LayerSpec(f"{name}_rank", 32, 1, c4.hidden, c4.inter, c4.num_loras, c4.lora_ranks,
                         lens, wi, seed=c4.seed, router="uniform_bias", pool_rank=c4.pool_rank)
    if name.endswith("_fp8") and name[:-4] in ("c1", "c3", "c4p", "c4d"):
        # the same layer and batch with fp8 e4m3 expert weights
        base = config(name[:-4])
        return dataclasses.replace(base, name=base.name + "_fp8", weights="fp8")
    raise KeyError(name)


CONFIG_NAMES = ("c0", "c1", "c2", "c3", "c4p", "c4d")
# the quantized-weight variants (fp8 e4m3 base weights, bf16 LoRA)
FP8_CONFIG_NAMES = ("c1_fp8", "c3_fp8", "c4p_fp8", "c4d_fp8")
# one rank's share of a layer under tensor / expert parallelism (shapes only)
SHARD_CONFIG_NAMES = ("c1_tp2", "c1_tp4", "c1_tp8", "c4p_ep8", "c4d_ep8")


# ----------------------------------------------------------------------------
# router (input generation only; the layer takes topk_ids / topk_weights)
# ----------------------------------------------------------------------------
def router_logits(spec: LayerSpec) -> np.ndarray:
    T, E = spec.num_tokens, spec.num_experts
    # c4p and c4d share the layer, hence the bias; the token logits differ per batch
    tok_key = 0 if spec.name.startswith("c4d") else 1
    rng = _rng(spec.seed, _TID_ROUTER, tok_key)
    if spec.router == "normal":
        return rng.standard_normal((T, E))
    if spec.router == "zipf":
        # popularity in softmax space ~ rank^-1.1 over a seeded permutation
        perm = _rng(spec.seed, _TID_BIAS).permutation(E) + 1
        bias = -1.1 * np.log(perm.astype(np.float64))
        return rng.standard_normal((T, E)) + bias[None, :]
    if spec.router == "uniform_bias":
        bias = _rng(spec.seed, _TID_BIAS).normal(0.0, np.sqrt(2.0), size=E)
        return rng.uniform(0.0, 1.0, size=(T, E)) + bias[None, :]
    raise ValueError(spec.router)


def route(logits: np.ndarray, k: int):
    """softmax -> top-k (ties to the lower expert id) -> renormalise."""
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    ids = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------
def quantize_fp8_blocks(w: torch.Tensor, block: int = 128, pow2: bool = False):
    """Input preparation for fp8 weights: a float [N, K] matrix as (OCP e4m3
    codes uint8 [N, K], float32 scales [N / block, K / block]) with
    scale = block amax / 448, or the next power of two up from it when
    ``pow2`` (1 for an all-zero block), and code = the e4m3 rounding of
    w / scale."""
    N, K = w.shape
    b = w.float().reshape(N // block, block, K // block, block)
    amax = b.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    if pow2:
        scale = torch.exp2(torch.ceil(torch.log2(scale)))
    q = (b / scale[:, None, :, None]).reshape(N, K).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def _randn(shape, std: float, seed: int, device, dtype) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def generate(spec: LayerSpec, device="cpu", canary: bool = True,
             with_lora: bool = True) -> Dict[str, object]:
    """Every input of the layer for ``spec`` as tensors on ``device``.

    Integer metadata is int32, router weights and scaling float32, the rest in
    ``spec.dtype``.  Returns a dict; ``meta`` holds the host copies of the
    request metadata.
    """
    dev = torch.device(device)
    dt = spec.torch_dtype
    T, E, k, H, I = spec.num_tokens, spec.num_experts, spec.top_k, spec.hidden, spec.inter
    L, R = spec.num_loras, spec.max_rank
    s = spec.seed

    seg_lens = np.asarray(spec.seg_lens, dtype=np.int64)
    seg_indptr = np.zeros(len(seg_lens) + 1, dtype=np.int32)
    seg_indptr[1:] = np.cumsum(seg_lens)
    wi = np.asarray(spec.weight_indices, dtype=np.int32)
    ranks = np.asarray(spec.lora_ranks, dtype=np.int32)
    scaling = np.full(L, spec.alpha_over_rank, dtype=np.float32)
    ids, w = route(router_logits(spec), k)

    out: Dict[str, object] = {}
    x_key = 0 if not spec.name.startswith("c4d") else 1
    out["x"] = _randn((T, H), 1.0, _subseed(s, _TID_X, x_key), dev, dt)
    if spec.weights in ("fp8", "fp8_f32scale"):
        pow2 = spec.weights == "fp8"
        if dt != torch.bfloat16:
            raise ValueError("fp8 expert weights go with bf16 activations")
        wgu = torch.empty((E, 2 * I, H), device=dev, dtype=torch.uint8)
        wd = torch.empty((E, H, I), device=dev, dtype=torch.uint8)
        sgu = torch.empty((E, 2 * I // 128, H // 128), device=dev, dtype=torch.float32)
        sd = torch.empty((E, H // 128, I // 128), device=dev, dtype=torch.float32)
        for e in range(E):
            wgu[e], sgu[e] = quantize_fp8_blocks(
                _randn((2 * I, H), 1.0 / np.sqrt(H), _subseed(s, _TID_WGU, e), dev, torch.float32),
                pow2=pow2)
            wd[e], sd[e] = quantize_fp8_blocks(
                _randn((H, I), 1.0 / np.sqrt(I), _subseed(s, _TID_WD, e), dev, torch.float32),
                pow2=pow2)
        out["w_gate_up_scale"], out["w_down_scale"] = sgu, sd
    else:
        wgu = torch.empty((E, 2 * I, H), device=dev, dtype=dt)
        wd = torch.empty((E, H, I), device=dev, dtype=dt)
        for e in range(E):
            wgu[e] = _randn((2 * I, H), 1.0 / np.sqrt(H), _subseed(s, _TID_WGU, e), dev, dt)
            wd[e] = _randn((H, I), 1.0 / np.sqrt(I), _subseed(s, _TID_WD, e), dev, dt)
    out["w_gate_up"], out["w_down"] = wgu, wd

    if with_lora and L > 0:
        fill = float("nan") if canary else 0.0
        pools = {}
        for name, tid, dim, std in (("a_gate", _TID_AG, H, 1.0 / np.sqrt(H)),
                                    ("a_up", _TID_AU, H, 1.0 / np.sqrt(H)),
                                    ("b_gate", _TID_BG, I, 0.1),
                                    ("b_up", _TID_BU, I, 0.1),
                                    ("a_down", _TID_AD, I, 1.0 / np.sqrt(I)),
                                    ("b_down", _TID_BD, H, 0.1)):
            pool = torch.full((L, E, R, dim), fill, device=dev, dtype=dt)
            for l in range(L):
                r = int(ranks[l])
                if r == 0:
                    continue
                # one draw per (pool, slot) covering every expert: a handful of
                # device launches per pool instead of one set per (slot, expert)
                pool[l, :, :r] = _randn((E, r, dim), std, _subseed(s, tid, l), dev, dt)
            pools[name] = pool
        out.update(pools)
    out["topk_ids"] = torch.from_numpy(ids).to(dev)
    out["topk_weights"] = torch.from_numpy(w).to(dev)
    out["seg_indptr"] = torch.from_numpy(seg_indptr).to(dev)
    out["weight_indices"] = torch.from_numpy(wi).to(dev)
    out["lora_ranks"] = torch.from_numpy(ranks).to(dev)
    out["scaling"] = torch.from_numpy(scaling).to(dev)
    out["meta"] = dict(seg_indptr=seg_indptr, weight_indices=wi, lora_ranks=ranks,
                       scaling=scaling, topk_ids=ids, topk_weights=w,
                       max_seg_len=int(seg_lens.max()) if len(seg_lens) else 0)
    return out


def random_spec(rng: np.random.Generator, *, max_experts=6, max_k=3, max_dim=96,
                max_loras=4, max_rank=8, max_reqs=5, max_len=6, dtype="f32",
                name="random") -> LayerSpec:
    """A small random layer (dims multiples of 8) for fuzz and property tests."""
    E = int(rng.integers(1, max_experts + 1))
    k = int(rng.integers(1, min(max_k, E) + 1))
    H = 8 * int(rng.integers(1, max_dim // 8 + 1))
    I = 8 * int(rng.integers(1, max_dim // 8 + 1))
    L = int(rng.integers(0, max_loras + 1))
    R = int(rng.integers(1, max_rank + 1))
    ranks = [int(v) for v in rng.integers(0, R + 1, size=L)]
    bs = int(rng.integers(1, max_reqs + 1))
    lens = [int(v) for v in rng.integers(0, max_len + 1, size=bs)]
    if sum(lens) == 0:
        lens[0] = 1
    wi = [int(v) for v in rng.integers(-1, L, size=bs)] if L > 0 else [-1] * bs
    return LayerSpec(name, E, k, H, I, L, ranks, lens, wi, dtype=dtype,
                     seed=int(rng.integers(0, 2**31)), router="normal", pool_rank=R)


# ----------------------------------------------------------------------------
# second workload: a dense projection with per-request LoRA and a two-slice
# output (the fused q_a_proj + kv_a_proj_with_mqa projection of MLA: outputs
# of 1536 and 512 + 64 columns over a 7168-wide hidden state)
# ----------------------------------------------------------------------------
_TID_DW, _TID_DA0, _TID_DA1, _TID_DB0, _TID_DB1 = 20, 21, 22, 23, 24


@dataclasses.dataclass
class DenseSpec:
    """One dense LoRA projection with outputs [0, out0) and [out0, out0 + out1)."""
    name: str
    hidden: int
    out0: int
    out1: int
    num_loras: int
    lora_ranks: List[int]
    seg_lens: List[int]
    weight_indices: List[int]
    dtype: str = "bf16"
    seed: int = 0
    alpha_over_rank: float = 2.0
    pool_rank: Optional[int] = None

    @property
    def num_tokens(self) -> int:
        return int(sum(self.seg_lens))

    @property
    def num_reqs(self) -> int:
        return len(self.seg_lens)

    @property
    def max_rank(self) -> int:
        if self.pool_rank is not None:
            return int(self.pool_rank)
        return max([int(r) for r in self.lora_ranks] + [1])

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def dense_config(name: str) -> DenseSpec:
    if name == "d0":
        return DenseSpec("d0_tiny_fp32", 256, 192, 64, 3, [8, 0, 16], [5, 1, 7, 3, 9],
                         [2, 0, -1, 1, 2], dtype="f32", seed=40, pool_rank=16)
    if name == "d1":
        # the Mixtral-prefill batch's request structure (16 requests, 4096 tokens, 8 slots of
        # rank 16 with slot 0 at rank 0, 2 requests without an adapter) on the MLA projection
        c1 = config("c1")
        return DenseSpec("d1_mla_qa_kva_prefill", 7168, 1536, 576, c1.num_loras, c1.lora_ranks,
                         c1.seg_lens, c1.weight_indices, seed=41, pool_rank=16)
    if name == "d2":
        return DenseSpec("d2_mla_qa_kva_decode", 7168, 1536, 576, 32, [32] * 32, [1] * 64,
                         [b % 32 for b in range(64)], seed=42, pool_rank=32)
    raise KeyError(name)


DENSE_CONFIG_NAMES = ("d0", "d1", "d2")


def generate_dense(spec: DenseSpec, device="cpu", canary: bool = True,
                   with_lora: bool = True) -> Dict[str, object]:
    """Every input of the dense LoRA projection for ``spec`` (same conventions as
    ``generate``: W ~ N(0, 1/H), A ~ N(0, 1/H), B ~ N(0, 0.01), rows past a
    slot's rank NaN when ``canary``)."""
    dev = torch.device(device)
    dt = spec.torch_dtype
    T, H, N0, N1 = spec.num_tokens, spec.hidden, spec.out0, spec.out1
    L, R, s = spec.num_loras, spec.max_rank, spec.seed
    seg_lens = np.asarray(spec.seg_lens, dtype=np.int64)
    seg_indptr = np.zeros(len(seg_lens) + 1, dtype=np.int32)
    seg_indptr[1:] = np.cumsum(seg_lens)
    wi = np.asarray(spec.weight_indices, dtype=np.int32)
    ranks = np.asarray(spec.lora_ranks, dtype=np.int32)
    scaling = np.full(L, spec.alpha_over_rank, dtype=np.float32)
    out: Dict[str, object] = {}
    out["x"] = _randn((T, H), 1.0, _subseed(s, _TID_X), dev, dt)
    out["w"] = _randn((N0 + N1, H), 1.0 / np.sqrt(H), _subseed(s, _TID_DW), dev, dt)
    if with_lora and L > 0:
        fill = float("nan") if canary else 0.0
        for name, tid, dim, std in (("a0", _TID_DA0, H, 1.0 / np.sqrt(H)),
                                    ("a1", _TID_DA1, H, 1.0 / np.sqrt(H)),
                                    ("b0", _TID_DB0, N0, 0.1), ("b1", _TID_DB1, N1, 0.1)):
            pool = torch.full((L, R, dim), fill, device=dev, dtype=dt)
            for l in range(L):
                r = int(ranks[l])
                if r > 0 and dim > 0:
                    pool[l, :r] = _randn((r, dim), std, _subseed(s, tid, l), dev, dt)
            out[name] = pool
    out["seg_indptr"] = torch.from_numpy(seg_indptr).to(dev)
    out["weight_indices"] = torch.from_numpy(wi).to(dev)
    out["lora_ranks"] = torch.from_numpy(ranks).to(dev)
    out["scaling"] = torch.from_numpy(scaling).to(dev)
    out["topk_ids"] = torch.zeros((T, 1), dtype=torch.int32, device=dev)
    out["meta"] = dict(seg_indptr=seg_indptr, weight_indices=wi, lora_ranks=ranks,
                       scaling=scaling, max_seg_len=int(seg_lens.max()) if len(seg_lens) else 0)
    return out
