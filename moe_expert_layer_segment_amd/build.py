"""Build the gfx950 MoE-LoRA shared library in-tree with hipcc.

    python -m moe_expert_layer_segment_amd.build

Produces ``moe_expert_layer_segment_amd/lib/libmoe_lora.so`` and its
``MOE_LORA_DEBUG`` twin ``lib/libmoe_lora_debug.so`` (the same kernels; info and
align additionally check their device-side preconditions and flag violations
in a device word).  Every HIP source is compiled for gfx950 only, with
packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoe_lora.so")
DEBUG_LIB = os.path.join(LIBDIR, "libmoe_lora_debug.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "route.hip", "info.hip", "align.hip", "forward.hip", "gemm_big.hip"]
# sources whose code differs under MOE_LORA_DEBUG (the rest is shared)
DEBUG_SOURCES = ["api.cpp", "info.hip", "align.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src: str, debug: bool = False) -> str:
    out = os.path.join(BUILD, ("debug_" if debug else "") + os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + (["-DMOE_LORA_DEBUG"] if debug else []) + \
        ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in DEBUG_SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    release = objs[:len(SOURCES)]
    debug = dict(zip(DEBUG_SOURCES, objs[len(SOURCES):]))
    _link(release, LIB)
    _link([debug.get(s, o) for s, o in zip(SOURCES, release)], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
