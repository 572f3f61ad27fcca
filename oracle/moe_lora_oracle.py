"""Plain, slow CPU oracle (numpy, float64) for the MoE-LoRA expert layer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code, tables or helpers with
the HIP path and imports nothing from it.

Sources (the pages are summaries of SGLang pull requests):

* the SGLang PR #14105 page (LoRA for MoE expert layers), section 实现拆解: the layer
  formula y = (W_down + (alpha/r) B_d A_d)[SiLU((W_gate + (alpha/r) B_g A_g) x)
  * ((W_up + (alpha/r) B_u A_u) x)], LoRA inserted after gate_up and before
  down; the align step sorts tokens by adapter and expert id; the LoRA pool is
  4-D [num_loras, num_experts, rank, dim].
* the SGLang PR #24160 page (sharing the MoE LoRA batch info), sections 实现拆解 and
  关键源码片段: per-batch metadata (seg_indptr, req_to_lora, adapter_enabled,
  token_lora_mapping with -1 = no adapter), the repeat_interleave / scatter
  closed forms of the unit test, the under-coverage assertion; section 评论区精华:
  -1 in weight_indices must be masked before the scatter.

Readings where the pages leave a step open (each is listed in the design notes):

* pools are rank-major: A as [L, E, R, in], B stored transposed as [L, E, R, out];
  the math B of the formula is ``pool_b[l, e, :r].T``;
* rows of a pool at index >= the slot's rank are never read;
* a pair carries LoRA iff its token's slot l >= 0, adapter_enabled[l] == 1 and
  lora_ranks[l] > 0;
* the top-k combine is y_t = sum_j w_tj * z_tj;
* under-coverage is an error iff max_seg_len > 0 and num_reqs * max_seg_len < T.

All floating point here is float64 on the exact values of the inputs.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


class UnderCoverError(AssertionError):
    """The launch described by (num_reqs, max_seg_len) under-covers tokens."""


# ---------------------------------------------------------------------------
# per-batch metadata (PR #24160 page, 实现拆解 items 1-3 and the unit test)
# ---------------------------------------------------------------------------
def moe_lora_info(num_tokens: int, seg_indptr, weight_indices, lora_ranks,
                  max_seg_len: int = 0):
    """Return (adapter_enabled int32[L], token_lora_mapping int32[T]).

    token_lora_mapping is weight_indices repeated over each request's segment
    (the repeat_interleave closed form of the unit test, -1 kept as "no
    adapter", per the MoELoRABatchInfo field comment).  adapter_enabled[i] is 1
    iff some request names slot i and lora_ranks[i] > 0 (the scatter closed
    form, with -1 masked out first as the review comment asks).
    """
    seg_indptr = np.asarray(seg_indptr, dtype=np.int64)
    wi = np.asarray(weight_indices, dtype=np.int64)
    ranks = np.asarray(lora_ranks, dtype=np.int64)
    bs, L = wi.shape[0], ranks.shape[0]
    if seg_indptr.shape[0] != bs + 1:
        raise ValueError("seg_indptr must have num_reqs + 1 entries")
    if seg_indptr[0] != 0 or seg_indptr[-1] != num_tokens or np.any(np.diff(seg_indptr) < 0):
        raise ValueError("seg_indptr must start at 0, be nondecreasing and end at num_tokens")
    if np.any(wi < -1) or np.any(wi >= L):
        raise ValueError("weight_indices must lie in [-1, num_loras)")
    if np.any(ranks < 0):
        raise ValueError("lora_ranks must be >= 0")
    if max_seg_len > 0 and bs * max_seg_len < num_tokens:
        raise UnderCoverError(
            f"launch under-covers tokens: {bs} requests x max_len {max_seg_len} < {num_tokens}")

    seg_lens = np.diff(seg_indptr)
    mapping = np.repeat(wi, seg_lens).astype(np.int32)

    enabled = np.zeros(L, dtype=np.int32)
    for b in range(bs):
        slot = wi[b]
        if slot >= 0:
            enabled[slot] = 1 if ranks[slot] > 0 else 0
    return enabled, mapping


# ---------------------------------------------------------------------------
# align: bucket (token, expert) pairs by (expert, adapter)
# (PR #14105 page, 实现拆解: tokens sorted by LoRA adapter and expert id)
# ---------------------------------------------------------------------------
def align_capacity_rows(num_pairs: int, num_experts: int, num_loras: int, block_m: int) -> int:
    """Upper bound of padded rows: every non-empty bucket adds < block_m pads."""
    nb = min(num_pairs, num_experts * (num_loras + 1))
    rows = num_pairs + nb * (block_m - 1)
    return ((rows + block_m - 1) // block_m) * block_m


def effective_adapter(token_lora_mapping, adapter_enabled) -> np.ndarray:
    """Slot of each token, or -1 when it has none or the slot is disabled."""
    m = np.asarray(token_lora_mapping, dtype=np.int64)
    en = np.asarray(adapter_enabled, dtype=np.int64)
    out = np.full(m.shape, -1, dtype=np.int64)
    for t in range(m.shape[0]):
        if m[t] >= 0 and en[m[t]] == 1:
            out[t] = m[t]
    return out


def moe_lora_align(topk_ids, token_lora_mapping, adapter_enabled, num_experts: int,
                   num_loras: int, block_m: int) -> Dict[str, np.ndarray]:
    """The canonical bucketed layout.

    Pair p = t*k + j has expert e = topk_ids[t, j] and effective slot a (the
    token's slot if enabled, else -1).  Buckets are keyed e*(L+1) + (a+1):
    expert-major, adapter-minor, the no-LoRA bucket first; inside a bucket pairs
    keep ascending p.  Each bucket is padded with the sentinel P up to a
    multiple of block_m, and every block_m rows form one tile labelled with the
    bucket's (e, a).  Unused capacity holds P / -1 / -1.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    P = T * k
    E, L, BM = num_experts, num_loras, block_m
    a_eff = effective_adapter(token_lora_mapping, adapter_enabled)

    keys = np.empty(P, dtype=np.int64)
    for p in range(P):
        t, j = divmod(p, k)
        e = ids[t, j]
        if not (0 <= e < E):
            raise ValueError("topk_ids out of range")
        keys[p] = e * (L + 1) + (a_eff[t] + 1)
    order = np.argsort(keys, kind="stable")  # ties by ascending p

    cap = align_capacity_rows(P, E, L, BM)
    sorted_ids = np.full(cap, P, dtype=np.int32)
    tile_expert = np.full(cap // BM, -1, dtype=np.int32)
    tile_lora = np.full(cap // BM, -1, dtype=np.int32)
    expert_tile_offsets = np.zeros(E + 1, dtype=np.int32)

    row = 0
    i = 0
    first_tile_of = {}
    while i < P:
        key = keys[order[i]]
        j = i
        while j < P and keys[order[j]] == key:
            j += 1
        e, a = divmod(int(key), L + 1)
        a -= 1
        n = j - i
        sorted_ids[row:row + n] = order[i:j]
        ntiles = (n + BM - 1) // BM
        t0 = row // BM
        tile_expert[t0:t0 + ntiles] = e
        tile_lora[t0:t0 + ntiles] = a
        first_tile_of.setdefault(e, t0)
        row += ntiles * BM
        i = j
    total_tiles = row // BM
    nxt = total_tiles
    for e in range(E - 1, -1, -1):
        if e in first_tile_of:
            nxt = first_tile_of[e]
        expert_tile_offsets[e] = nxt
    expert_tile_offsets[E] = total_tiles
    return dict(sorted_pair_ids=sorted_ids, tile_expert=tile_expert, tile_lora=tile_lora,
                expert_tile_offsets=expert_tile_offsets,
                num_rows_padded=np.array([row], dtype=np.int32))


# ---------------------------------------------------------------------------
# forward (PR #14105 page, 实现拆解: the layer formula)
# ---------------------------------------------------------------------------
def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v))."""
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _lora_on(l: int, adapter_enabled, lora_ranks) -> bool:
    return l >= 0 and int(adapter_enabled[l]) == 1 and int(lora_ranks[l]) > 0


def moe_lora_forward(x, topk_ids, topk_weights, w_gate_up, w_down,
                     lora_ranks, scaling, token_lora_mapping, adapter_enabled,
                     a_gate=None, a_up=None, b_gate=None, b_up=None,
                     a_down=None, b_down=None,
                     tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """y[t] = sum_j w[t,j] * (W_down' [SiLU(W_gate' x_t) * (W_up' x_t)]) with
    W' = W[e] + s_l * B[l,e] A[l,e] for the token's slot l when LoRA is on.

    The LoRA term is applied in factored form, s * (x A^T) B^T, with
    A = pool_a[l, e, :r] and B^T = pool_b[l, e, :r]; it equals the merged form
    by associativity.  Pairs are grouped by expert, then by slot, so that each
    product is a plain matmul over the pairs of that group.

    Weights and pools may be any objects supporting ``[e]`` / ``[l, e]`` that
    yield array-likes (e.g. a lazy per-expert view).  ``tokens`` restricts the
    computation to a subset; the result then has one row per listed token.
    Returns float64 [len(tokens), H].
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = _f64(topk_weights)
    mapping = np.asarray(token_lora_mapping, dtype=np.int64)
    ranks = np.asarray(lora_ranks, dtype=np.int64)
    scal = _f64(scaling)
    T, k = ids.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    H = np.asarray(x[0]).shape[-1] if T > 0 else 0
    y = np.zeros((tok.shape[0], H), dtype=np.float64)
    if tok.shape[0] == 0:
        return y
    have_lora = a_gate is not None and ranks.shape[0] > 0

    # pairs restricted to the selected tokens: (row in y, token, slot j)
    row_of = np.repeat(np.arange(tok.shape[0]), k)
    t_of = np.repeat(tok, k)
    j_of = np.tile(np.arange(k), tok.shape[0])
    e_of = ids[t_of, j_of]
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        X = _f64(np.stack([np.asarray(x[t]) for t in t_of[sel]]))
        wgu = _f64(w_gate_up[int(e)])
        I = wgu.shape[0] // 2
        wg, wu = wgu[:I], wgu[I:]
        wd = _f64(w_down[int(e)])
        g = X @ wg.T
        u = X @ wu.T
        slots = mapping[t_of[sel]]
        if have_lora:
            for l in np.unique(slots):
                if not _lora_on(int(l), adapter_enabled, ranks):
                    continue
                r, s = int(ranks[l]), scal[l]
                m = slots == l
                ag = _f64(a_gate[int(l), int(e)])[:r]
                au = _f64(a_up[int(l), int(e)])[:r]
                bg = _f64(b_gate[int(l), int(e)])[:r]
                bu = _f64(b_up[int(l), int(e)])[:r]
                g[m] += s * ((X[m] @ ag.T) @ bg)
                u[m] += s * ((X[m] @ au.T) @ bu)
        act = silu(g) * u
        z = act @ wd.T
        if have_lora:
            for l in np.unique(slots):
                if not _lora_on(int(l), adapter_enabled, ranks):
                    continue
                r, s = int(ranks[l]), scal[l]
                m = slots == l
                ad = _f64(a_down[int(l), int(e)])[:r]
                bd = _f64(b_down[int(l), int(e)])[:r]
                z[m] += s * ((act[m] @ ad.T) @ bd)
        wsel = w[t_of[sel], j_of[sel]]
        y[row_of[sel]] += wsel[:, None] * z
    return y


def moe_lora_forward_bruteforce(x, topk_ids, topk_weights, w_gate_up, w_down,
                                lora_ranks, scaling, token_lora_mapping, adapter_enabled,
                                a_gate=None, a_up=None, b_gate=None, b_up=None,
                                a_down=None, b_down=None) -> np.ndarray:
    """The closed form, token by token: merge W' = W + s * B A for each
    (token, expert) pair, then apply the SwiGLU expert and the top-k weighted
    sum.  Pure Python loops; for tiny inputs only."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = _f64(topk_weights)
    mapping = np.asarray(token_lora_mapping, dtype=np.int64)
    ranks = np.asarray(lora_ranks, dtype=np.int64)
    scal = _f64(scaling)
    T, k = ids.shape
    X = _f64(x)
    H = X.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    have_lora = a_gate is not None and ranks.shape[0] > 0
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            wgu = _f64(w_gate_up[e])
            I = wgu.shape[0] // 2
            Wg, Wu, Wd = wgu[:I].copy(), wgu[I:].copy(), _f64(w_down[e]).copy()
            l = int(mapping[t])
            if have_lora and _lora_on(l, adapter_enabled, ranks):
                r, s = int(ranks[l]), scal[l]
                Bg = _f64(b_gate[l, e])[:r].T      # [I, r]
                Bu = _f64(b_up[l, e])[:r].T        # [I, r]
                Bd = _f64(b_down[l, e])[:r].T      # [H, r]
                Wg = Wg + s * (Bg @ _f64(a_gate[l, e])[:r])
                Wu = Wu + s * (Bu @ _f64(a_up[l, e])[:r])
                Wd = Wd + s * (Bd @ _f64(a_down[l, e])[:r])
            gate = Wg @ X[t]
            up = Wu @ X[t]
            a = silu(gate) * up
            y[t] += w[t, j] * (Wd @ a)
    return y


# ---------------------------------------------------------------------------
# router (the layer configs: softmax over the experts, top-k, renormalised)
# ---------------------------------------------------------------------------
def moe_lora_route(logits, top_k: int):
    """Return (topk_ids int32[T, k], topk_weights float64[T, k]).

    Each token keeps the k experts of largest softmax probability, in
    descending order with ties to the lower expert id, and their weights are
    renormalised over the k.

    Softmax is strictly increasing in the logit, so the ranking is the ranking
    of the logits themselves, taken on the exact input values (fp64
    probabilities of very negative logits can underflow to equal values and
    would break ties differently).  In the renormalised weight the softmax
    normaliser cancels: w_j = exp(l_j - m) / sum over the k of exp(l_i - m),
    with m the largest logit.
    """
    lg = np.asarray(logits, dtype=np.float64)
    if lg.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = lg.shape
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    expert = np.arange(E)
    for t in range(T):
        # primary key: descending logit; secondary: ascending expert id
        order = np.lexsort((expert, -lg[t]))[:top_k]
        ids[t] = order
        top = lg[t, order]
        e = np.exp(top - top[0])
        w[t] = e / e.sum()
    return ids, w


# ---------------------------------------------------------------------------
# fp8 expert weights (the quantized-MoE-LoRA variant: fp8 base weights, bf16
# LoRA).  Format: OCP 8-bit floating point, E4M3 -- 1 sign bit, 4 exponent
# bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
# m * 2^-9; no infinities; S.1111.111 is NaN, so the largest finite value is
# 1.75 * 2^8 = 448.  Block scaling: weight (e, n, k) = code * scale[e, n / 128,
# k / 128] over 128 x 128 blocks of each expert's [rows, K] matrix.
# ---------------------------------------------------------------------------
def decode_e4m3(codes) -> np.ndarray:
    """float64 values of OCP E4M3 codes (uint8 array of any shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = man * 2.0 ** -9
    v = sign * np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def dequantize_block_fp8(codes, scales, block: int = 128) -> np.ndarray:
    """float64 weights from E4M3 codes [..., N, K] and block scales
    [..., N / block, K / block]: each code times the scale of its block."""
    w = decode_e4m3(codes)
    s = np.asarray(scales, dtype=np.float64)
    n, k = w.shape[-2], w.shape[-1]
    if n % block or k % block or s.shape[-2:] != (n // block, k // block):
        raise ValueError("codes and scales do not tile into blocks")
    s_full = np.repeat(np.repeat(s, block, axis=-2), block, axis=-1)
    return w * s_full


# ---------------------------------------------------------------------------
# dense projection with a two-slice LoRA output (PR #22323 page, sections
# 功能与动机 and 实现拆解 item 2: the fused q_a_proj + kv_a_proj_with_mqa
# projection of MLA, outputs of unequal size, LoRA B split in two and applied
# per output part).  Reading: each output slice i has its own LoRA factors
# (A_i, B_i); the slot of a token and its masking are those of the MoE layer.
# ---------------------------------------------------------------------------
def dense_lora_forward(x, w, n0: int, lora_ranks, scaling, token_lora_mapping,
                       adapter_enabled, a0=None, a1=None, b0=None, b1=None,
                       tokens=None) -> np.ndarray:
    """y [T, N0 + N1] float64:
    y[t, :N0] = x_t W[:N0]^T + on_t s_l (x_t A0[l, :r]^T) B0[l, :r]
    y[t, N0:] = x_t W[N0:]^T + on_t s_l (x_t A1[l, :r]^T) B1[l, :r]
    with B stored transposed (rank-major, [L, R, out]) and on_t as in
    moe_lora_forward.  ``tokens``: compute only these rows (same order)."""
    X = _f64(x)
    W = _f64(w)
    T = X.shape[0]
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    X = X[rows]
    y = X @ W.T
    N0 = int(n0)
    mapping = np.asarray(token_lora_mapping, dtype=np.int64)[rows]
    ranks = np.asarray(lora_ranks, dtype=np.int64)
    scal = np.asarray(scaling, dtype=np.float64)
    if a0 is None or len(ranks) == 0:
        return y
    for l in np.unique(mapping):
        l = int(l)
        if not _lora_on(l, adapter_enabled, ranks):
            continue
        m = mapping == l
        r, s = int(ranks[l]), scal[l]
        y[m, :N0] += s * ((X[m] @ _f64(a0[l])[:r].T) @ _f64(b0[l])[:r])
        if y.shape[1] > N0:
            y[m, N0:] += s * ((X[m] @ _f64(a1[l])[:r].T) @ _f64(b1[l])[:r])
    return y
