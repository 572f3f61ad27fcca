"""Compile-time checks of the gfx950 kernels (no GPU needed): no kernel keeps
registers or private arrays in scratch memory, and the GEMM kernels fit two
waves per SIMD.  A silent spill or a register array left dynamically indexed
costs an order of magnitude in run time without changing results.

The large-tile GEMM runs at the edge of the register file (128 accumulator
registers per lane plus its operand fragments); there the check is that its K
loop -- the loop holding the barrier between K tiles -- touches no scratch,
and that the few values parked outside it stay few."""
import os
import re
import shutil
import subprocess

import pytest

from moe_expert_layer_segment_amd import build as B

HAVE_HIPCC = shutil.which(B.hipcc()) is not None or os.path.exists(B.hipcc())


def _resources(src, tmp_path):
    cmd = [B.hipcc()] + B.common_flags() + ["-c", os.path.join(B.CSRC, src), "-o",
                                            str(tmp_path / "k.o"),
                                            "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels = re.split(r"remark: Function Name: ", out)[1:]
    assert kernels, "no resource report"
    res = {}
    for rep in kernels:
        name = rep.split()[0]
        res[name] = dict(
            scratch=int(re.search(r"ScratchSize \[bytes/lane\]: (\d+)", rep).group(1)),
            spill=int(re.search(r"VGPRs Spill: (\d+)", rep).group(1)),
            occ=int(re.search(r"Occupancy \[waves/SIMD\]: (\d+)", rep).group(1)))
    return res


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc missing")
@pytest.mark.parametrize("src", ["forward.hip", "align.hip", "info.hip", "route.hip"])
def test_kernels_use_no_scratch(src, tmp_path):
    for name, r in _resources(src, tmp_path).items():
        assert r["scratch"] == 0 and r["spill"] == 0, (name, r)
        if "gemm_kernel" in name:
            assert r["occ"] >= 2, (name, r)


def _k_loop_scratch(asm, kernel):
    """Scratch instructions inside the K loop of `kernel` in hipcc -S output:
    of the loops whose body holds the barrier after the all-loads wait, the
    innermost one with the MFMAs (another serves waves whose rows all lie past
    a short item's end, and the persistent tile loop holds them all)."""
    start = asm.index(kernel + ":")
    body = asm[start:asm.index("s_endpgm", start)].split("\n")
    labels = {l.split(":")[0].strip(): i for i, l in enumerate(body) if l.startswith(".LBB")}
    loops = []
    for bar in (i for i, l in enumerate(body) if "s_waitcnt vmcnt(0) lgkmcnt(0)" in l):
        for i in range(bar, len(body)):
            tok = body[i].split()
            if tok and tok[0].startswith("s_cbranch") and tok[-1] in labels and labels[tok[-1]] < bar:
                loops.append(body[labels[tok[-1]]:i + 1])
                break
    with_mfma = [lp for lp in loops if sum("v_mfma" in l for l in lp) >= 32]
    assert with_mfma, "K loop not found"
    k_loop = min(with_mfma, key=len)
    return sum("scratch_" in l for l in k_loop)


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc missing")
def test_large_tile_gemm_k_loop_has_no_spills(tmp_path):
    res = _resources("gemm_big.hip", tmp_path)
    assert len(res) == 2
    for name, r in res.items():
        assert r["occ"] >= 2 and r["spill"] <= 64, (name, r)
    asm_path = tmp_path / "k.s"
    subprocess.run([B.hipcc()] + B.common_flags() + ["--cuda-device-only", "-S",
                                                    os.path.join(B.CSRC, "gemm_big.hip"), "-o",
                                                    str(asm_path)], check=True, capture_output=True)
    asm = asm_path.read_text()
    for name in res:
        assert _k_loop_scratch(asm, name) == 0, name
