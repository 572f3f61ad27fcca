"""Compile-time checks of the gfx950 kernels (no GPU needed): no kernel keeps
registers or private arrays in scratch memory, and the GEMM kernels fit two
waves per SIMD.  A silent spill or a register array left dynamically indexed
costs an order of magnitude in run time without changing results."""
import os
import re
import shutil
import subprocess

import pytest

from moe_expert_layer_segment_amd import build as B


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                    reason="hipcc missing")
@pytest.mark.parametrize("src", ["forward.hip", "align.hip", "info.hip"])
def test_kernels_use_no_scratch(src, tmp_path):
    cmd = [B.hipcc()] + B.common_flags() + ["-c", os.path.join(B.CSRC, src), "-o",
                                            str(tmp_path / "k.o"),
                                            "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels = re.split(r"remark: Function Name: ", out)[1:]
    assert kernels, "no resource report"
    for rep in kernels:
        name = rep.split()[0]
        scratch = int(re.search(r"ScratchSize \[bytes/lane\]: (\d+)", rep).group(1))
        spill = int(re.search(r"VGPRs Spill: (\d+)", rep).group(1))
        assert scratch == 0 and spill == 0, (name, scratch, spill)
        if "gemm_kernel" in name:
            occ = int(re.search(r"Occupancy \[waves/SIMD\]: (\d+)", rep).group(1))
            assert occ >= 2, (name, occ)
