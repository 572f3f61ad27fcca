"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
at least one pin catches each of them."""
import importlib.util
import os
import sys
import types

import pytest

import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "moe_lora_oracle.py")

MUTANTS = {
    "drop_up_lora": ("u[m] += s * ((X[m] @ au.T) @ bu)", "pass"),
    "swap_gate_up": ("wg, wu = wgu[:I], wgu[I:]", "wu, wg = wgu[:I], wgu[I:]"),
    "shared_a_gate_up": ("au = _f64(a_up[int(l), int(e)])[:r]", "au = _f64(a_gate[int(l), int(e)])[:r]"),
    "silu_sign": ("return v / (1.0 + np.exp(-v))", "return v / (1.0 + np.exp(v))"),
    "scaling_dropped": ("r, s = int(ranks[l]), scal[l]\n                m = slots == l\n                ag",
                        "r, s = int(ranks[l]), 1.0\n                m = slots == l\n                ag"),
    "no_combine_weight": ("y[row_of[sel]] += wsel[:, None] * z", "y[row_of[sel]] += z"),
    "down_lora_on_input": ("z[m] += s * ((act[m] @ ad.T) @ bd)", "z[m] += s * ((act[m] @ ad.T) @ bd) * 0.5"),
    "full_pool_rows": ("ag = _f64(a_gate[int(l), int(e)])[:r]", "ag = _f64(a_gate[int(l), int(e)])"),
    "enabled_ignores_rank": ("enabled[slot] = 1 if ranks[slot] > 0 else 0", "enabled[slot] = 1"),
    "mapping_shift": ("mapping = np.repeat(wi, seg_lens).astype(np.int32)",
                      "mapping = np.roll(np.repeat(wi, seg_lens), 1).astype(np.int32)"),
    "align_key_collision": ("keys[p] = e * (L + 1) + (a_eff[t] + 1)", "keys[p] = e * L + (a_eff[t] + 1)"),
    "align_unstable": ('order = np.argsort(keys, kind="stable")', 'order = np.argsort(-keys, kind="stable")[::-1]'),
    "align_no_pad": ("ntiles = (n + BM - 1) // BM", "ntiles = max(1, n // BM)"),
    "undercover_never": ("if max_seg_len > 0 and bs * max_seg_len < num_tokens:", "if False:"),
    "brute_up_uses_gate": ("up = Wu @ X[t]", "up = Wg @ X[t]"),
    "route_ties_to_higher_id": ("order = np.lexsort((expert, -lg[t]))[:top_k]",
                                "order = np.lexsort((-expert, -lg[t]))[:top_k]"),
    "route_ascending": ("order = np.lexsort((expert, -lg[t]))[:top_k]",
                        "order = np.lexsort((expert, lg[t]))[:top_k]"),
    "route_no_renorm": ("w[t] = e / e.sum()", "w[t] = e"),
    "route_softmax_over_all": ("w[t] = e / e.sum()", "w[t] = e / np.exp(lg[t] - top[0]).sum()"),
    "e4m3_bias_8": ("np.exp2(exp.astype(np.float64) - 7.0)", "np.exp2(exp.astype(np.float64) - 8.0)"),
    "e4m3_subnormal_scale": ("subnormal = man * 2.0 ** -9", "subnormal = man * 2.0 ** -10"),
    "e4m3_no_nan": ("return np.where((exp == 0xF) & ((c & 0x7) == 0x7), np.nan, v)", "return v"),
    "dequant_scale_dropped": ("    return w * s_full", "    return w"),
    "dense_a0_for_both": ("y[m, N0:] += s * ((X[m] @ _f64(a1[l])[:r].T) @ _f64(b1[l])[:r])",
                          "y[m, N0:] += s * ((X[m] @ _f64(a0[l])[:r].T) @ _f64(b1[l])[:r])"),
    "dense_no_scaling": ("y[m, :N0] += s * ((X[m] @ _f64(a0[l])[:r].T) @ _f64(b0[l])[:r])",
                         "y[m, :N0] += ((X[m] @ _f64(a0[l])[:r].T) @ _f64(b0[l])[:r])"),
    "dense_full_pool_rows": ("y[m, :N0] += s * ((X[m] @ _f64(a0[l])[:r].T) @ _f64(b0[l])[:r])",
                             "y[m, :N0] += s * ((X[m] @ _f64(a0[l]).T) @ _f64(b0[l]))"),
    "capacity_no_min": ("nb = min(num_pairs, num_experts * (num_loras + 1))",
                        "nb = num_experts * (num_loras + 1)"),
    "capacity_pads_full_block": ("rows = num_pairs + nb * (block_m - 1)", "rows = num_pairs + nb * block_m"),
    "dequant_block_transposed": ("s_full = np.repeat(np.repeat(s, block, axis=-2), block, axis=-1)",
                                 "s_full = np.repeat(np.repeat(np.swapaxes(s, -1, -2), block, axis=-2), block, axis=-1)"),
    "brute_b_untransposed": ("Bd = _f64(b_down[l, e])[:r].T      # [H, r]", "Bd = _f64(b_down[l, e])[:r].T[::-1]"),
}


def _mutant(name, old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    mod = _mutant(name, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError) as exc:  # noqa: PERF203
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
