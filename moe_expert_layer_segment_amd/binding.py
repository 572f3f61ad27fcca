"""ctypes binding of the gfx950 MoE-LoRA library (argument marshalling only).

Every step of the layer runs in the HIP kernels behind ``include/moe_lora.h``;
this module only checks tensor shapes / dtypes / devices, allocates outputs and
workspaces with PyTorch, and passes raw device pointers and the current HIP
stream.  If the shared library is missing it raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LORA_LIB") or os.path.join(_PKG, "lib", "libmoe_lora.so")
# the same library built with MOE_LORA_DEBUG (device-side precondition checks)
DEBUG_LIB_PATH = os.path.join(_PKG, "lib", "libmoe_lora_debug.so")

OK, ERR_INVALID, ERR_UNDERCOVER, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4, -5
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
_FP8_TORCH = (torch.uint8, torch.float8_e4m3fn)   # one-byte e4m3 codes
FORWARD_STAGES = ("plan", "shrink_gate_up", "gate_up_gemm", "shrink_down", "down_gemm", "combine")

_c_i32p = ctypes.POINTER(ctypes.c_int32)


class ForwardArgs(ctypes.Structure):
    """Mirror of ``moe_lora_forward_args``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("dtype", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("num_loras", ctypes.c_int32),
        ("max_rank", ctypes.c_int32), ("block_m", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
        ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("a_gate", ctypes.c_void_p), ("a_up", ctypes.c_void_p), ("b_gate", ctypes.c_void_p),
        ("b_up", ctypes.c_void_p), ("a_down", ctypes.c_void_p), ("b_down", ctypes.c_void_p),
        ("lora_ranks", ctypes.c_void_p), ("scaling", ctypes.c_void_p),
        ("sorted_pair_ids", ctypes.c_void_p), ("tile_expert", ctypes.c_void_p),
        ("tile_lora", ctypes.c_void_p), ("expert_tile_offsets", ctypes.c_void_p),
        ("num_rows_padded", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("y", ctypes.c_void_p), ("out_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
        ("w_gate_up_scale", ctypes.c_void_p), ("w_down_scale", ctypes.c_void_p),
    ]


_LIB = None
_DEBUG_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        _LIB = _load(LIB_PATH)
    return _LIB


def debug_lib() -> ctypes.CDLL:
    """The MOE_LORA_DEBUG build of the library (same calls, same results; info
    and align also flag device-side precondition violations, read with
    ``moe_lora_debug_flags``)."""
    global _DEBUG_LIB
    if _DEBUG_LIB is None:
        _DEBUG_LIB = _load(DEBUG_LIB_PATH)
    return _DEBUG_LIB


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"MoE-LoRA HIP library not found at {path}; build it with "
            "`python -m moe_expert_layer_segment_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(path)
    L.moe_lora_status_str.restype = ctypes.c_char_p
    L.moe_lora_status_str.argtypes = [ctypes.c_int]
    L.moe_lora_route.restype = ctypes.c_int
    L.moe_lora_route.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 4
    L.moe_lora_info.restype = ctypes.c_int
    L.moe_lora_info.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 6
    L.moe_lora_align_capacity_rows.restype = ctypes.c_int64
    L.moe_lora_align_capacity_rows.argtypes = [ctypes.c_int32] * 5
    L.moe_lora_align_workspace_bytes.restype = ctypes.c_size_t
    L.moe_lora_align_workspace_bytes.argtypes = [ctypes.c_int32] * 5
    L.moe_lora_align.restype = ctypes.c_int
    L.moe_lora_align.argtypes = ([ctypes.c_int32] * 5 + [ctypes.c_void_p] * 9 +
                                 [ctypes.c_size_t, ctypes.c_void_p])
    L.moe_lora_forward_workspace_bytes.restype = ctypes.c_size_t
    L.moe_lora_forward_workspace_bytes.argtypes = [ctypes.POINTER(ForwardArgs)]
    L.moe_lora_forward.restype = ctypes.c_int
    L.moe_lora_forward.argtypes = [ctypes.POINTER(ForwardArgs), ctypes.c_void_p]
    L.moe_lora_forward_events.restype = ctypes.c_int
    L.moe_lora_forward_events.argtypes = [ctypes.POINTER(ForwardArgs), ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_void_p)]
    L.moe_lora_dense_workspace_bytes.restype = ctypes.c_size_t
    L.moe_lora_dense_workspace_bytes.argtypes = [ctypes.POINTER(DenseArgs)]
    L.moe_lora_dense_forward.restype = ctypes.c_int
    L.moe_lora_dense_forward.argtypes = [ctypes.POINTER(DenseArgs), ctypes.c_void_p]
    L.moe_lora_dense_forward_events.restype = ctypes.c_int
    L.moe_lora_dense_forward_events.argtypes = [ctypes.POINTER(DenseArgs), ctypes.c_void_p,
                                                ctypes.POINTER(ctypes.c_void_p)]
    L.moe_lora_forward_noalloc.restype = ctypes.c_int
    L.moe_lora_forward_noalloc.argtypes = [ctypes.POINTER(ForwardArgs), ctypes.c_void_p]
    L.moe_lora_forward_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
    L.moe_lora_forward_noalloc_max_workspace_bytes.argtypes = []
    L.moe_lora_debug_flags.restype = ctypes.c_int
    L.moe_lora_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                                       ctypes.c_void_p]
    return L


DEBUG_SEG_INDPTR, DEBUG_WEIGHT_INDEX, DEBUG_RANK, DEBUG_EXPERT_ID, DEBUG_MAPPING = 1, 2, 4, 8, 16


def debug_flags(clear: bool = True, library: Optional[ctypes.CDLL] = None) -> int:
    """The precondition flag word of a MOE_LORA_DEBUG build (after synchronising
    the current stream); ``clear`` resets it."""
    L = library or debug_lib()
    v = ctypes.c_uint32(0)
    _check(L.moe_lora_debug_flags(ctypes.byref(v), int(clear), _stream()), "moe_lora_debug_flags")
    return int(v.value)


class MoeLoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib().moe_lora_status_str(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str):
    if status == ERR_UNDERCOVER:
        # the pages' unit test expects an AssertionError naming under-coverage
        raise AssertionError(f"{where}: launch under-covers tokens")
    if status != OK:
        raise MoeLoraError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {t.numel()}")


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------
def moe_lora_route(logits: torch.Tensor, top_k: int, topk_ids: Optional[torch.Tensor] = None,
                   topk_weights: Optional[torch.Tensor] = None):
    """(topk_ids int32 [T, k], topk_weights fp32 [T, k]) from fp32 router logits [T, E]."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _need(topk_ids, "topk_ids", torch.int32, logits.device, T * top_k)
    _need(topk_weights, "topk_weights", torch.float32, logits.device, T * top_k)
    _check(lib().moe_lora_route(T, E, top_k, _ptr(logits), _ptr(topk_ids), _ptr(topk_weights),
                                _stream()), "moe_lora_route")
    return topk_ids, topk_weights


# ---------------------------------------------------------------------------
# info
# ---------------------------------------------------------------------------
def moe_lora_info(num_tokens: int, seg_indptr: torch.Tensor, lora_ranks: torch.Tensor,
                  weight_indices: torch.Tensor, adapter_enabled: Optional[torch.Tensor] = None,
                  token_lora_mapping: Optional[torch.Tensor] = None, max_len: int = 0):
    """Per-batch metadata; returns (adapter_enabled, token_lora_mapping[:num_tokens]).

    Argument order follows the pages' ``_compute_moe_lora_info``.  Preallocated
    outputs are written in place and returned as views of the same storage.
    Raises AssertionError when num_reqs * max_len < num_tokens.
    """
    dev = seg_indptr.device
    num_reqs = seg_indptr.numel() - 1
    num_loras = lora_ranks.numel()
    _need(seg_indptr, "seg_indptr", torch.int32)
    _need(lora_ranks, "lora_ranks", torch.int32, dev)
    _need(weight_indices, "weight_indices", torch.int32, dev, num_reqs)
    if adapter_enabled is None:
        adapter_enabled = torch.empty(num_loras, dtype=torch.int32, device=dev)
    if token_lora_mapping is None:
        token_lora_mapping = torch.empty(max(num_tokens, 1), dtype=torch.int32, device=dev)
    _need(adapter_enabled, "adapter_enabled", torch.int32, dev, num_loras)
    _need(token_lora_mapping, "token_lora_mapping", torch.int32, dev, num_tokens)
    st = lib().moe_lora_info(num_tokens, num_reqs, num_loras, int(max_len), _ptr(seg_indptr),
                             _ptr(weight_indices), _ptr(lora_ranks), _ptr(adapter_enabled),
                             _ptr(token_lora_mapping), _stream())
    _check(st, "moe_lora_info")
    return adapter_enabled, token_lora_mapping[:num_tokens]


compute_moe_lora_info = moe_lora_info


# ---------------------------------------------------------------------------
# align
# ---------------------------------------------------------------------------
def moe_lora_align_capacity_rows(num_tokens, top_k, num_experts, num_loras, block_m) -> int:
    v = lib().moe_lora_align_capacity_rows(num_tokens, top_k, num_experts, num_loras, block_m)
    if v < 0:
        raise MoeLoraError(ERR_INVALID, "moe_lora_align_capacity_rows")
    return int(v)


def moe_lora_align_workspace_bytes(num_tokens, top_k, num_experts, num_loras, block_m) -> int:
    return int(lib().moe_lora_align_workspace_bytes(num_tokens, top_k, num_experts, num_loras,
                                                    block_m))


def moe_lora_align(topk_ids: torch.Tensor, token_lora_mapping: torch.Tensor,
                   adapter_enabled: Optional[torch.Tensor], num_experts: int, num_loras: int,
                   block_m: int = 16, out: Optional[Dict[str, torch.Tensor]] = None,
                   workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Bucket (token, expert) pairs by (expert, adapter); returns the align outputs."""
    dev = topk_ids.device
    T, k = topk_ids.shape
    _need(topk_ids, "topk_ids", torch.int32)
    _need(token_lora_mapping, "token_lora_mapping", torch.int32, dev, T)
    if num_loras > 0:
        _need(adapter_enabled, "adapter_enabled", torch.int32, dev, num_loras)
    cap = moe_lora_align_capacity_rows(T, k, num_experts, num_loras, block_m)
    if out is None:
        out = dict(
            sorted_pair_ids=torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
            tile_expert=torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
            tile_lora=torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
            expert_tile_offsets=torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
            num_rows_padded=torch.empty(1, dtype=torch.int32, device=dev))
    for name, n in (("sorted_pair_ids", cap), ("tile_expert", cap // block_m),
                    ("tile_lora", cap // block_m), ("expert_tile_offsets", num_experts + 1),
                    ("num_rows_padded", 1)):
        _need(out[name], name, torch.int32, dev, n)
    wsb = moe_lora_align_workspace_bytes(T, k, num_experts, num_loras, block_m)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, wsb)
    st = lib().moe_lora_align(T, k, num_experts, num_loras, block_m, _ptr(topk_ids),
                              _ptr(token_lora_mapping),
                              _ptr(adapter_enabled) if num_loras > 0 else None,
                              _ptr(out["sorted_pair_ids"]), _ptr(out["tile_expert"]),
                              _ptr(out["tile_lora"]), _ptr(out["expert_tile_offsets"]),
                              _ptr(out["num_rows_padded"]), _ptr(workspace), workspace.numel(),
                              _stream())
    _check(st, "moe_lora_align")
    out["capacity"] = cap
    out["block_m"] = block_m
    return out


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
_POOLS = ("a_gate", "a_up", "b_gate", "b_up", "a_down", "b_down")


def _forward_args(x, topk_weights, w_gate_up, w_down, align_out, lora_ranks, scaling, pools,
                  top_k, y, workspace, out_dtype=None, w_scales=None) -> ForwardArgs:
    T, H = x.shape
    E, twoI, H2 = w_gate_up.shape
    I = twoI // 2
    if x.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif x.dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    dev = x.device
    _need(x, "x", x.dtype)
    fp8 = w_gate_up.dtype in _FP8_TORCH
    wdt = w_gate_up.dtype if fp8 else x.dtype
    _need(w_gate_up, "w_gate_up", wdt, dev)
    _need(w_down, "w_down", wdt, dev)
    if H2 != H or tuple(w_down.shape) != (E, H, I):
        raise ValueError("weight shapes do not match x / each other")
    if fp8:
        if x.dtype != torch.bfloat16:
            raise TypeError("fp8 expert weights need bf16 activations")
        if w_scales is None:
            raise ValueError("fp8 expert weights need their block scales (w_scales)")
        sgu, sd = w_scales
        _need(sgu, "w_gate_up_scale", torch.float32, dev)
        _need(sd, "w_down_scale", torch.float32, dev)
        if tuple(sgu.shape) != (E, 2 * I // 128, H // 128) or tuple(sd.shape) != (E, H // 128, I // 128):
            raise ValueError("block scales must be [E, 2I/128, H/128] and [E, H/128, I/128]")
    _need(topk_weights, "topk_weights", torch.float32, dev, T * top_k)
    L, R = 0, 0
    if pools is not None:
        L, E2, R, _ = pools["a_gate"].shape
        if E2 != E:
            raise ValueError("pool expert axis does not match the weights")
        shapes = dict(a_gate=(L, E, R, H), a_up=(L, E, R, H), b_gate=(L, E, R, I),
                      b_up=(L, E, R, I), a_down=(L, E, R, I), b_down=(L, E, R, H))
        for n in _POOLS:
            _need(pools[n], n, x.dtype, dev)
            if tuple(pools[n].shape) != shapes[n]:
                raise ValueError(f"{n} must have shape {shapes[n]}, got {tuple(pools[n].shape)}")
        _need(lora_ranks, "lora_ranks", torch.int32, dev, L)
        _need(scaling, "scaling", torch.float32, dev, L)
    a = ForwardArgs()
    a.struct_size = ctypes.sizeof(ForwardArgs)
    a.dtype = dt
    out_dt = x.dtype if out_dtype is None else out_dtype
    if out_dt == torch.float32:
        a.out_dtype = DTYPE_F32
    elif out_dt == x.dtype:
        a.out_dtype = dt
    else:
        raise TypeError(f"unsupported output dtype {out_dt}")
    a.num_tokens, a.hidden, a.inter, a.num_experts, a.top_k = T, H, I, E, top_k
    a.num_loras, a.max_rank, a.block_m = L, R, int(align_out["block_m"])
    a.x, a.topk_weights = x.data_ptr(), topk_weights.data_ptr()
    a.w_gate_up, a.w_down = w_gate_up.data_ptr(), w_down.data_ptr()
    if fp8:
        a.weight_dtype = DTYPE_FP8_E4M3
        a.w_gate_up_scale, a.w_down_scale = w_scales[0].data_ptr(), w_scales[1].data_ptr()
    if pools is not None:
        for n in _POOLS:
            setattr(a, n, pools[n].data_ptr())
        a.lora_ranks, a.scaling = lora_ranks.data_ptr(), scaling.data_ptr()
    for n in ("sorted_pair_ids", "tile_expert", "tile_lora", "expert_tile_offsets",
              "num_rows_padded"):
        _need(align_out[n], n, torch.int32, dev)
        setattr(a, n, align_out[n].data_ptr())
    if y is not None:
        _need(y, "y", out_dt, dev, T * H)
        a.y = y.data_ptr()
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return a


def moe_lora_forward_workspace_bytes(x, topk_weights, w_gate_up, w_down, align_out, top_k,
                                     lora_ranks=None, scaling=None, pools=None,
                                     w_scales=None) -> int:
    a = _forward_args(x, topk_weights, w_gate_up, w_down, align_out, lora_ranks, scaling, pools,
                      top_k, None, None, w_scales=w_scales)
    n = int(lib().moe_lora_forward_workspace_bytes(ctypes.byref(a)))
    if n == 0:
        raise MoeLoraError(ERR_INVALID, "moe_lora_forward_workspace_bytes")
    return n


def moe_lora_forward(x: torch.Tensor, topk_weights: torch.Tensor, w_gate_up: torch.Tensor,
                     w_down: torch.Tensor, align_out: Dict[str, torch.Tensor], top_k: int,
                     lora_ranks: Optional[torch.Tensor] = None,
                     scaling: Optional[torch.Tensor] = None,
                     pools: Optional[Dict[str, torch.Tensor]] = None,
                     y: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     events=None, out_dtype=None, w_scales=None) -> torch.Tensor:
    """The MoE-LoRA layer: returns y [T, H] (written into ``y`` if given).

    fp8 expert weights: ``w_gate_up`` / ``w_down`` as uint8 or float8_e4m3fn
    e4m3 codes and ``w_scales`` = (gate_up scales [E, 2I/128, H/128], down
    scales [E, H/128, I/128]), float32.

    ``events``: optional sequence of 2 * len(FORWARD_STAGES) raw hipEvent_t
    handles recorded around each kernel stage (measurement only).
    """
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype if out_dtype is None else out_dtype,
                        device=x.device)
    if workspace is None:
        n = moe_lora_forward_workspace_bytes(x, topk_weights, w_gate_up, w_down, align_out, top_k,
                                             lora_ranks, scaling, pools, w_scales)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    a = _forward_args(x, topk_weights, w_gate_up, w_down, align_out, lora_ranks, scaling, pools,
                      top_k, y, workspace, out_dtype, w_scales)
    if events is None:
        _check(lib().moe_lora_forward(ctypes.byref(a), _stream()), "moe_lora_forward")
    else:
        if len(events) != 2 * len(FORWARD_STAGES):
            raise ValueError("events needs one pair per forward stage")
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(lib().moe_lora_forward_events(ctypes.byref(a), _stream(), arr),
               "moe_lora_forward_events")
    return y


def moe_lora_forward_noalloc(x: torch.Tensor, topk_weights: torch.Tensor, w_gate_up: torch.Tensor,
                             w_down: torch.Tensor, align_out: Dict[str, torch.Tensor], top_k: int,
                             lora_ranks: Optional[torch.Tensor] = None,
                             scaling: Optional[torch.Tensor] = None,
                             pools: Optional[Dict[str, torch.Tensor]] = None,
                             y: Optional[torch.Tensor] = None, out_dtype=None,
                             w_scales=None) -> torch.Tensor:
    """moe_lora_forward without a caller workspace: the library's static
    per-device scratch serves instead (problems up to
    ``moe_lora_forward_noalloc_max_workspace_bytes()``; calls on one device must
    not overlap).  Only ``y`` is allocated here, and only when not given."""
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype if out_dtype is None else out_dtype,
                        device=x.device)
    a = _forward_args(x, topk_weights, w_gate_up, w_down, align_out, lora_ranks, scaling, pools,
                      top_k, y, None, out_dtype, w_scales)
    _check(lib().moe_lora_forward_noalloc(ctypes.byref(a), _stream()), "moe_lora_forward_noalloc")
    return y


def moe_lora_forward_noalloc_max_workspace_bytes() -> int:
    return int(lib().moe_lora_forward_noalloc_max_workspace_bytes())


def run_layer(inputs: dict, block_m: int = 16, with_lora: bool = True,
              out_dtype=None) -> torch.Tensor:
    """info -> align -> forward on a dict from ``workloads.generate``."""
    T = inputs["x"].shape[0]
    k = inputs["topk_ids"].shape[1]
    E = inputs["w_gate_up"].shape[0]
    L = inputs["lora_ranks"].numel() if with_lora and "a_gate" in inputs else 0
    ranks = inputs["lora_ranks"]
    en, mp = moe_lora_info(T, inputs["seg_indptr"], ranks, inputs["weight_indices"],
                           max_len=inputs["meta"]["max_seg_len"])
    al = moe_lora_align(inputs["topk_ids"], mp, en if L > 0 else None, E, L, block_m)
    pools = {n: inputs[n] for n in _POOLS} if L > 0 else None
    ws = ((inputs["w_gate_up_scale"], inputs["w_down_scale"])
          if "w_gate_up_scale" in inputs else None)
    return moe_lora_forward(inputs["x"], inputs["topk_weights"], inputs["w_gate_up"],
                            inputs["w_down"], al, k, ranks if L > 0 else None,
                            inputs["scaling"] if L > 0 else None, pools, out_dtype=out_dtype,
                            w_scales=ws)


# ---------------------------------------------------------------------------
# dense projection with a two-slice LoRA output
# ---------------------------------------------------------------------------
DENSE_STAGES = ("plan", "shrink", "gemm", "combine")


class DenseArgs(ctypes.Structure):
    """Mirror of ``moe_lora_dense_args``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("dtype", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("out0", ctypes.c_int32),
        ("out1", ctypes.c_int32), ("num_loras", ctypes.c_int32), ("max_rank", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("a0", ctypes.c_void_p), ("a1", ctypes.c_void_p), ("b0", ctypes.c_void_p),
        ("b1", ctypes.c_void_p),
        ("lora_ranks", ctypes.c_void_p), ("scaling", ctypes.c_void_p),
        ("sorted_pair_ids", ctypes.c_void_p), ("tile_expert", ctypes.c_void_p),
        ("tile_lora", ctypes.c_void_p), ("expert_tile_offsets", ctypes.c_void_p),
        ("num_rows_padded", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("y", ctypes.c_void_p), ("out_dtype", ctypes.c_int32),
    ]


def _dense_args(x, w, out0, align_out, lora_ranks, scaling, pools, y, workspace,
                out_dtype=None) -> DenseArgs:
    T, H = x.shape
    N, H2 = w.shape
    if H2 != H or not (0 < out0 <= N):
        raise ValueError("w must be [out0 + out1, H] with 0 < out0 <= its rows")
    if x.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif x.dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    dev = x.device
    _need(x, "x", x.dtype)
    _need(w, "w", x.dtype, dev)
    out1 = N - out0
    L, R = 0, 0
    if pools is not None:
        L, R, _ = pools["a0"].shape
        shapes = dict(a0=(L, R, H), a1=(L, R, H), b0=(L, R, out0), b1=(L, R, out1))
        for n in ("a0", "b0") + (("a1", "b1") if out1 > 0 else ()):
            _need(pools[n], n, x.dtype, dev)
            if tuple(pools[n].shape) != shapes[n]:
                raise ValueError(f"{n} must have shape {shapes[n]}, got {tuple(pools[n].shape)}")
        _need(lora_ranks, "lora_ranks", torch.int32, dev, L)
        _need(scaling, "scaling", torch.float32, dev, L)
    a = DenseArgs()
    a.struct_size = ctypes.sizeof(DenseArgs)
    a.dtype = dt
    out_dt = x.dtype if out_dtype is None else out_dtype
    if out_dt == torch.float32:
        a.out_dtype = DTYPE_F32
    elif out_dt == x.dtype:
        a.out_dtype = dt
    else:
        raise TypeError(f"unsupported output dtype {out_dt}")
    a.num_tokens, a.hidden, a.out0, a.out1 = T, H, out0, out1
    a.num_loras, a.max_rank, a.block_m = L, R, int(align_out["block_m"])
    a.x, a.w = x.data_ptr(), w.data_ptr()
    if pools is not None:
        a.a0, a.b0 = pools["a0"].data_ptr(), pools["b0"].data_ptr()
        if out1 > 0:
            a.a1, a.b1 = pools["a1"].data_ptr(), pools["b1"].data_ptr()
        a.lora_ranks, a.scaling = lora_ranks.data_ptr(), scaling.data_ptr()
    for n in ("sorted_pair_ids", "tile_expert", "tile_lora", "expert_tile_offsets",
              "num_rows_padded"):
        _need(align_out[n], n, torch.int32, dev)
        setattr(a, n, align_out[n].data_ptr())
    if y is not None:
        _need(y, "y", out_dt, dev, T * N)
        a.y = y.data_ptr()
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return a


def moe_lora_dense_workspace_bytes(x, w, out0, align_out, lora_ranks=None, scaling=None,
                                   pools=None) -> int:
    a = _dense_args(x, w, out0, align_out, lora_ranks, scaling, pools, None, None)
    n = int(lib().moe_lora_dense_workspace_bytes(ctypes.byref(a)))
    if n == 0:
        raise MoeLoraError(ERR_INVALID, "moe_lora_dense_workspace_bytes")
    return n


def moe_lora_dense_forward(x: torch.Tensor, w: torch.Tensor, out0: int,
                           align_out: Dict[str, torch.Tensor],
                           lora_ranks: Optional[torch.Tensor] = None,
                           scaling: Optional[torch.Tensor] = None,
                           pools: Optional[Dict[str, torch.Tensor]] = None,
                           y: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           events=None, out_dtype=None) -> torch.Tensor:
    """Dense projection with per-request LoRA and two output slices: y [T, N]
    (``pools``: a0, a1 [L, R, H], b0 [L, R, out0], b1 [L, R, N - out0]).
    ``align_out`` comes from moe_lora_align with one expert and top_k = 1."""
    T = x.shape[0]
    N = w.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=x.dtype if out_dtype is None else out_dtype, device=x.device)
    if workspace is None:
        n = moe_lora_dense_workspace_bytes(x, w, out0, align_out, lora_ranks, scaling, pools)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    a = _dense_args(x, w, out0, align_out, lora_ranks, scaling, pools, y, workspace, out_dtype)
    if events is None:
        _check(lib().moe_lora_dense_forward(ctypes.byref(a), _stream()), "moe_lora_dense_forward")
    else:
        if len(events) != 2 * len(DENSE_STAGES):
            raise ValueError("events needs one pair per dense stage")
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(lib().moe_lora_dense_forward_events(ctypes.byref(a), _stream(), arr),
               "moe_lora_dense_forward_events")
    return y


def run_dense(inputs: dict, out0: int, block_m: int = 16, with_lora: bool = True,
              out_dtype=None) -> torch.Tensor:
    """info -> align (one expert, top_k = 1) -> dense forward on a dict from
    ``workloads.generate_dense``."""
    T = inputs["x"].shape[0]
    L = inputs["lora_ranks"].numel() if with_lora and "a0" in inputs else 0
    ranks = inputs["lora_ranks"]
    en, mp = moe_lora_info(T, inputs["seg_indptr"], ranks, inputs["weight_indices"],
                           max_len=inputs["meta"]["max_seg_len"])
    al = moe_lora_align(inputs["topk_ids"], mp, en if L > 0 else None, 1, L, block_m)
    pools = {n: inputs[n] for n in ("a0", "a1", "b0", "b1")} if L > 0 else None
    return moe_lora_dense_forward(inputs["x"], inputs["w"], out0, al, ranks if L > 0 else None,
                                  inputs["scaling"] if L > 0 else None, pools,
                                  out_dtype=out_dtype)
