"""The MOE_LORA_DEBUG build: info and align flag device-side precondition
violations in a device word (the page on sharing the MoE LoRA batch info,
section 评论区精华: a -1 slot index must not reach the scatter unchecked),
while giving the same outputs as the release build.  Every invalid input here
stays in bounds of the kernels' buffers (the release kernels ignore such
values), so nothing can fault."""
import ctypes

import pytest
import torch

from gpu_helpers import say
from moe_expert_layer_segment_amd import binding

pytestmark = pytest.mark.gpu

I32 = torch.int32


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _info(dl, T, seg, wi, ranks):
    L = ranks.numel()
    en = torch.full((max(L, 1),), -7, dtype=I32, device="cuda")
    mp = torch.full((max(T, 1),), -7, dtype=I32, device="cuda")
    st = dl.moe_lora_info(T, seg.numel() - 1, L, 0, _p(seg), _p(wi), _p(ranks), _p(en), _p(mp),
                          binding._stream())
    assert st == binding.OK
    return en, mp


def _align(dl, ids, mp, en, E, L, BM=16):
    T, k = ids.shape
    cap = binding.moe_lora_align_capacity_rows(T, k, E, L, BM)
    out = [torch.empty(cap, dtype=I32, device="cuda"), torch.empty(cap // BM, dtype=I32, device="cuda"),
           torch.empty(cap // BM, dtype=I32, device="cuda"), torch.empty(E + 1, dtype=I32, device="cuda"),
           torch.empty(1, dtype=I32, device="cuda")]
    wsb = binding.moe_lora_align_workspace_bytes(T, k, E, L, BM)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    st = dl.moe_lora_align(T, k, E, L, BM, _p(ids), _p(mp), _p(en), *[_p(o) for o in out], _p(ws),
                           wsb, binding._stream())
    assert st == binding.OK
    return out


def test_debug_flags_on_invalid_inputs():
    dl = binding.debug_lib()
    binding.debug_flags(clear=True)
    say("debug build: valid inputs raise no flag")
    seg = torch.tensor([0, 3, 3, 7], dtype=I32, device="cuda")
    wi = torch.tensor([1, -1, 0], dtype=I32, device="cuda")
    ranks = torch.tensor([8, 16], dtype=I32, device="cuda")
    en, mp = _info(dl, 7, seg, wi, ranks)
    ids = torch.tensor([[0, 1], [2, 3], [1, 0], [3, 2], [0, 2], [1, 3], [2, 0]], dtype=I32, device="cuda")
    good = _align(dl, ids, mp, en, 4, 2)
    assert binding.debug_flags() == 0
    # the debug build's outputs equal the release build's
    en_r, mp_r = binding.moe_lora_info(7, seg, ranks, wi)
    al_r = binding.moe_lora_align(ids, mp_r, en_r, 4, 2, 16)
    assert torch.equal(en, en_r[:2]) and torch.equal(mp[:7], mp_r)
    for o, n in zip(good, ("sorted_pair_ids", "tile_expert", "tile_lora", "expert_tile_offsets",
                           "num_rows_padded")):
        assert torch.equal(o, al_r[n]), n
    assert binding.debug_flags() == 0

    say("debug build: each precondition flagged on its own")
    cases = [
        (torch.tensor([0, 4, 3, 7], dtype=I32, device="cuda"), wi, ranks, binding.DEBUG_SEG_INDPTR),
        (torch.tensor([1, 3, 3, 7], dtype=I32, device="cuda"), wi, ranks, binding.DEBUG_SEG_INDPTR),
        (torch.tensor([0, 3, 3, 6], dtype=I32, device="cuda"), wi, ranks, binding.DEBUG_SEG_INDPTR),
        (seg, torch.tensor([1, 2, 0], dtype=I32, device="cuda"), ranks, binding.DEBUG_WEIGHT_INDEX),
        (seg, torch.tensor([1, -2, 0], dtype=I32, device="cuda"), ranks, binding.DEBUG_WEIGHT_INDEX),
        (seg, wi, torch.tensor([8, -1], dtype=I32, device="cuda"), binding.DEBUG_RANK),
    ]
    for s, w, r, bit in cases:
        _info(dl, 7, s, w, r)
        assert binding.debug_flags() == bit, bit
    bad_ids = ids.clone()
    bad_ids[4, 1] = 4          # expert id == E: dropped by align, flagged here
    _align(dl, bad_ids, mp, en, 4, 2)
    assert binding.debug_flags() == binding.DEBUG_EXPERT_ID
    bad_ids[4, 1] = -3
    _align(dl, bad_ids, mp, en, 4, 2)
    assert binding.debug_flags() == binding.DEBUG_EXPERT_ID
    bad_mp = mp.clone()
    bad_mp[2] = 2              # slot == L
    _align(dl, ids, bad_mp, en, 4, 2)
    assert binding.debug_flags() == binding.DEBUG_MAPPING
    # flags accumulate until read; clear=False keeps them
    _info(dl, 7, seg, torch.tensor([1, 5, 0], dtype=I32, device="cuda"), torch.tensor([8, -1], dtype=I32, device="cuda"))
    assert binding.debug_flags(clear=False) == binding.DEBUG_WEIGHT_INDEX | binding.DEBUG_RANK
    assert binding.debug_flags() == binding.DEBUG_WEIGHT_INDEX | binding.DEBUG_RANK
    assert binding.debug_flags() == 0
