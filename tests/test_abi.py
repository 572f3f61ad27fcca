"""The C ABI without a GPU: the library loads, exports every function the header
declares, the ctypes struct mirrors the C struct, and host-side validation
returns the documented status codes before touching any device memory."""
import ctypes
import os
import re
import subprocess

import pytest

from moe_expert_layer_segment_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_lora.h")


def _declared_functions():
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_lora_[a-z_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("moe_lora_info", "moe_lora_align", "moe_lora_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


def test_forward_args_layout_matches_c(tmp_path):
    fields = [f[0] for f in binding.ForwardArgs._fields_]
    prog = tmp_path / "layout.c"
    body = "\n".join(
        f'  printf("{n} %zu\\n", offsetof(moe_lora_forward_args, {n}));' for n in fields)
    prog.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"moe_lora.h\"\n"
        "int main(void) {\n"
        '  printf("size %zu\\n", sizeof(moe_lora_forward_args));\n' + body + "\n  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(line.split() for line in out if line.strip())
    assert int(got["size"]) == ctypes.sizeof(binding.ForwardArgs)
    for n in fields:
        assert int(got[n]) == getattr(binding.ForwardArgs, n).offset, n


def test_header_compiles_as_c_and_cpp(tmp_path):
    for comp, ext in (("gcc", "c"), ("g++", "cpp")):
        src = tmp_path / f"inc.{ext}"
        src.write_text('#include "moe_lora.h"\nint main(void) { return MOE_LORA_OK; }\n')
        subprocess.run([comp, "-I", os.path.join(ROOT, "include"), "-c", str(src), "-o",
                        str(tmp_path / f"inc_{ext}.o")], check=True)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_status_strings():
    lib = binding.lib()
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert lib.moe_lora_status_str(st)


def test_info_validation_codes():
    lib = binding.lib()
    f = lib.moe_lora_info
    assert f(-1, 1, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(5, 0, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID
    # the pages' under-coverage example: one request of 300 tokens, max_len 1
    assert f(300, 1, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == binding.ERR_UNDERCOVER
    assert f(4, 1, 1, 0, None, FAKE, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(4, 1, 1, 0, FAKE, FAKE, None, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(0, 0, 0, 0, FAKE, None, None, None, None, None) == binding.OK


def test_route_validation_codes():
    lib = binding.lib()
    f = lib.moe_lora_route
    assert f(-1, 8, 2, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(4, 0, 1, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(4, 8, 0, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(4, 8, 9, FAKE, FAKE, FAKE, None) == binding.ERR_INVALID       # top_k > E
    assert f(4, 64, 17, FAKE, FAKE, FAKE, None) == binding.ERR_UNSUPPORTED  # top_k > 16
    assert f(4, 8, 2, None, FAKE, FAKE, None) == binding.ERR_INVALID
    assert f(4, 8, 2, FAKE, None, FAKE, None) == binding.ERR_INVALID
    assert f(4, 8, 2, FAKE, FAKE, None, None) == binding.ERR_INVALID
    assert f(0, 8, 2, None, None, None, None) == binding.OK                 # nothing enqueued


def test_align_validation_codes():
    lib = binding.lib()
    f = lib.moe_lora_align
    args = [FAKE] * 8
    assert f(4, 2, 8, 2, 15, *args, FAKE, 1 << 30, None) == binding.ERR_INVALID  # block_m
    assert f(4, 2, 8, 2, 512, *args, FAKE, 1 << 30, None) == binding.ERR_INVALID
    assert f(4, 9, 8, 2, 16, *args, FAKE, 1 << 30, None) == binding.ERR_INVALID  # k > E
    assert f(4, 2, 8, 5000, 16, *args, FAKE, 1 << 30, None) == binding.ERR_UNSUPPORTED
    assert f(4, 2, 8, 2, 16, *args, FAKE, 1, None) == binding.ERR_WORKSPACE
    assert f(4, 2, 8, 2, 16, *args, None, 1 << 30, None) == binding.ERR_WORKSPACE
    assert lib.moe_lora_align_capacity_rows(4, 2, 8, 2, 16) == 16 * ((8 + 8 * 15 + 15) // 16)
    assert lib.moe_lora_align_capacity_rows(4, 2, 8, 2, 17) == -1
    assert lib.moe_lora_align_workspace_bytes(4, 2, 8, 2, 16) > 0


def _fargs(**over):
    a = binding.ForwardArgs()
    a.struct_size = ctypes.sizeof(binding.ForwardArgs)
    a.dtype = binding.DTYPE_BF16
    a.num_tokens, a.hidden, a.inter, a.num_experts, a.top_k = 8, 128, 256, 4, 2
    a.num_loras, a.max_rank, a.block_m = 2, 16, 16
    for n, _ in binding.ForwardArgs._fields_:
        if n not in ("struct_size", "dtype", "num_tokens", "hidden", "inter", "num_experts",
                     "top_k", "num_loras", "max_rank", "block_m", "workspace_bytes",
                     "out_dtype", "weight_dtype"):
            setattr(a, n, 0x1000)
    a.workspace_bytes = 1
    a.out_dtype = binding.DTYPE_BF16
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_forward_validation_codes():
    lib = binding.lib()
    call = lambda **o: lib.moe_lora_forward(ctypes.byref(_fargs(**o)), None)  # noqa: E731
    assert call(dtype=7) == binding.ERR_UNSUPPORTED
    assert call(out_dtype=5) == binding.ERR_UNSUPPORTED
    assert call(out_dtype=binding.DTYPE_F32) == binding.ERR_WORKSPACE  # fp32 output is allowed
    assert call(struct_size=8) == binding.ERR_INVALID
    assert call(hidden=100) == binding.ERR_UNSUPPORTED
    assert call(max_rank=65) == binding.ERR_UNSUPPORTED
    assert call(top_k=5) == binding.ERR_INVALID
    assert call(block_m=24) == binding.ERR_INVALID
    assert call(x=None) == binding.ERR_INVALID
    assert call(a_down=None) == binding.ERR_INVALID
    # 16-byte units: a misaligned activation, weight, pool, output or workspace is refused
    for n in ("x", "w_gate_up", "w_down", "b_gate", "b_down", "a_up", "y", "workspace"):
        assert call(**{n: 0x1008}) == binding.ERR_INVALID, n
    assert call(num_loras=0, b_down=0x1002) == binding.ERR_WORKSPACE   # pools unused
    assert call() == binding.ERR_WORKSPACE           # 1-byte workspace
    assert call(num_loras=0, a_gate=None) == binding.ERR_WORKSPACE  # plain MoE needs no pools
    ws = lib.moe_lora_forward_workspace_bytes(ctypes.byref(_fargs()))
    assert ws > 0
    # sizing needs no pointers at all
    bare = _fargs()
    for n, _ in binding.ForwardArgs._fields_:
        if n not in ("struct_size", "dtype", "num_tokens", "hidden", "inter", "num_experts",
                     "top_k", "num_loras", "max_rank", "block_m", "workspace_bytes",
                     "out_dtype", "weight_dtype"):
            setattr(bare, n, None)
    assert lib.moe_lora_forward_workspace_bytes(ctypes.byref(bare)) == ws
    assert lib.moe_lora_forward_workspace_bytes(ctypes.byref(_fargs(dtype=9))) == 0
    assert call(num_tokens=0) == binding.OK


def test_forward_fp8_weight_validation():
    lib = binding.lib()
    call = lambda **o: lib.moe_lora_forward(ctypes.byref(_fargs(**o)), None)  # noqa: E731
    F8 = binding.DTYPE_FP8_E4M3
    # H = 128, I = 256: valid fp8 shapes (the 1-byte workspace is the only error)
    assert call(weight_dtype=F8) == binding.ERR_WORKSPACE
    assert call(weight_dtype=binding.DTYPE_BF16) == binding.ERR_WORKSPACE   # same as dtype
    assert call(weight_dtype=F8, dtype=binding.DTYPE_F32, out_dtype=binding.DTYPE_F32) == \
        binding.ERR_UNSUPPORTED                                             # fp8 needs bf16 x
    assert call(weight_dtype=F8, hidden=192) == binding.ERR_UNSUPPORTED     # H % 128
    assert call(weight_dtype=F8, inter=320) == binding.ERR_UNSUPPORTED      # I % 128
    assert call(weight_dtype=F8, hidden=16384 + 128) == binding.ERR_UNSUPPORTED
    assert call(weight_dtype=3) == binding.ERR_UNSUPPORTED
    assert call(weight_dtype=F8, w_down_scale=None) == binding.ERR_INVALID
    assert call(weight_dtype=F8, w_gate_up_scale=None) == binding.ERR_INVALID
    assert call(weight_dtype=F8, w_gate_up_scale=None, num_tokens=0) == binding.OK
    # a caller whose struct ends at out_dtype gets weights in dtype
    old = binding.ForwardArgs.out_dtype.offset + 4          # the struct before the fp8 fields
    assert call(struct_size=old, weight_dtype=3) == binding.ERR_WORKSPACE
    assert call(struct_size=old + 4, weight_dtype=3) == binding.ERR_WORKSPACE   # with its padding
    assert call(struct_size=old - 4) == binding.ERR_INVALID
    # fp8 weights need no buffer beyond the bf16 layout (which also holds the
    # partial sums of split gate_up tail tiles, unused with fp8 weights)
    ws8 = lib.moe_lora_forward_workspace_bytes(ctypes.byref(_fargs(weight_dtype=F8)))
    assert 0 < ws8 <= lib.moe_lora_forward_workspace_bytes(ctypes.byref(_fargs()))


def _dargs(**over):
    a = binding.DenseArgs()
    a.struct_size = ctypes.sizeof(binding.DenseArgs)
    a.dtype = binding.DTYPE_BF16
    a.num_tokens, a.hidden, a.out0, a.out1 = 8, 128, 192, 64
    a.num_loras, a.max_rank, a.block_m = 2, 16, 16
    for n, _ in binding.DenseArgs._fields_:
        if n not in ("struct_size", "dtype", "num_tokens", "hidden", "out0", "out1", "num_loras",
                     "max_rank", "block_m", "workspace_bytes", "out_dtype"):
            setattr(a, n, 0x1000)
    a.workspace_bytes = 1
    a.out_dtype = binding.DTYPE_BF16
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_dense_validation_codes():
    lib = binding.lib()
    call = lambda **o: lib.moe_lora_dense_forward(ctypes.byref(_dargs(**o)), None)  # noqa: E731
    assert call() == binding.ERR_WORKSPACE                     # valid but a 1-byte workspace
    assert call(dtype=7) == binding.ERR_UNSUPPORTED
    assert call(out_dtype=binding.DTYPE_F32) == binding.ERR_WORKSPACE
    assert call(struct_size=8) == binding.ERR_INVALID
    assert call(out0=0) == binding.ERR_INVALID
    assert call(out1=-64) == binding.ERR_INVALID
    assert call(out0=100) == binding.ERR_UNSUPPORTED
    assert call(out1=96) == binding.ERR_UNSUPPORTED
    assert call(hidden=100) == binding.ERR_UNSUPPORTED
    assert call(max_rank=65) == binding.ERR_UNSUPPORTED
    assert call(block_m=24) == binding.ERR_INVALID
    assert call(w=None) == binding.ERR_INVALID
    assert call(b1=None) == binding.ERR_INVALID
    for n in ("x", "w", "b0", "a1", "y", "workspace"):
        assert call(**{n: 0x1004}) == binding.ERR_INVALID, n   # 16-byte units
    assert call(out1=0, a1=None, b1=None) == binding.ERR_WORKSPACE   # one slice needs no second pool
    assert call(num_loras=0, a0=None, b0=None, a1=None, b1=None) == binding.ERR_WORKSPACE
    assert call(num_tokens=0) == binding.OK
    ws = lib.moe_lora_dense_workspace_bytes(ctypes.byref(_dargs()))
    assert ws > 0 and lib.moe_lora_dense_workspace_bytes(ctypes.byref(_dargs(dtype=9))) == 0


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        binding.moe_lora_info(3, torch.tensor([0, 3], dtype=torch.int32),
                              torch.tensor([4], dtype=torch.int32),
                              torch.tensor([0], dtype=torch.int32))


def test_size_limits_of_32bit_offsets():
    """x [T, H] and one expert's weight matrix are addressed with 32-bit byte
    offsets from 64-bit bases: sizes reaching 4 GiB are refused before launch."""
    lib = binding.lib()
    call = lambda **o: lib.moe_lora_forward(ctypes.byref(_fargs(**o)), None)  # noqa: E731
    ws = lambda **o: lib.moe_lora_forward_workspace_bytes(ctypes.byref(_fargs(**o)))  # noqa: E731
    # bf16 x of 2^20 tokens x 2048 = 4 GiB: refused; one token fewer is accepted
    assert call(num_tokens=1 << 20, top_k=1, hidden=2048) == binding.ERR_UNSUPPORTED
    assert ws(num_tokens=1 << 20, top_k=1, hidden=2048) == 0
    assert call(num_tokens=(1 << 20) - 1, top_k=1, hidden=2048) == binding.ERR_WORKSPACE
    # fp32 halves the token limit
    f32 = dict(dtype=binding.DTYPE_F32, out_dtype=binding.DTYPE_F32)
    assert call(num_tokens=1 << 19, top_k=1, hidden=2048, **f32) == binding.ERR_UNSUPPORTED
    # one expert's gate_up matrix: 2 * I * H * 2 bytes < 4 GiB
    assert call(hidden=32768, inter=32768) == binding.ERR_UNSUPPORTED
    assert call(hidden=16384, inter=32768) == binding.ERR_WORKSPACE
    # the dense projection: x and w likewise
    dcall = lambda **o: lib.moe_lora_dense_forward(ctypes.byref(_dargs(**o)), None)  # noqa: E731
    assert dcall(num_tokens=1 << 20, hidden=2048) == binding.ERR_UNSUPPORTED
    assert dcall(hidden=65536, out0=32768, out1=0, a1=None, b1=None) == binding.ERR_UNSUPPORTED


def test_dense_ctypes_signatures_return_size_t():
    """The dense sizing call returns a size_t: without a declared restype ctypes
    would truncate it to a C int above 2 GiB."""
    lib = binding.lib()
    assert lib.moe_lora_dense_workspace_bytes.restype is ctypes.c_size_t
    assert lib.moe_lora_forward_workspace_bytes.restype is ctypes.c_size_t
    # a large dense batch (8M tokens x 2048 bf16 outputs: the fp32 partials alone are 64 GiB)
    big = lib.moe_lora_dense_workspace_bytes(ctypes.byref(_dargs(num_tokens=1 << 23, hidden=128,
                                                                 out0=2048, out1=0, a1=None,
                                                                 b1=None)))
    assert big > (1 << 34)


def test_release_build_has_no_debug_checks():
    """moe_lora_debug_flags exists in every build; a release build reports
    UNSUPPORTED (and 0) without touching a device."""
    lib = binding.lib()
    v = ctypes.c_uint32(77)
    assert lib.moe_lora_debug_flags(ctypes.byref(v), 1, None) == binding.ERR_UNSUPPORTED
    assert v.value == 0
    assert lib.moe_lora_debug_flags(None, 1, None) == binding.ERR_INVALID


def test_debug_build_exports_every_declared_symbol():
    dl = binding.debug_lib()
    missing = [n for n in _declared_functions() if not hasattr(dl, n)]
    assert not missing, missing


def test_noalloc_forward_refuses_oversized_problems():
    """The allocation-free forward serves problems whose workspace fits its
    static scratch; a larger one is refused before any device call."""
    lib = binding.lib()
    cap = lib.moe_lora_forward_noalloc_max_workspace_bytes()
    assert cap == 64 << 20
    big = _fargs(num_tokens=4096, hidden=4096, inter=14336, num_experts=8)
    assert lib.moe_lora_forward_workspace_bytes(ctypes.byref(big)) > cap
    assert lib.moe_lora_forward_noalloc(ctypes.byref(big), None) == binding.ERR_WORKSPACE
    # argument errors come first, as for moe_lora_forward; the workspace fields are ignored
    assert lib.moe_lora_forward_noalloc(ctypes.byref(_fargs(dtype=7)), None) == binding.ERR_UNSUPPORTED
    assert lib.moe_lora_forward_noalloc(ctypes.byref(_fargs(x=None)), None) == binding.ERR_INVALID
    assert lib.moe_lora_forward_noalloc(ctypes.byref(_fargs(x=0x1008)), None) == binding.ERR_INVALID
    assert lib.moe_lora_forward_noalloc(ctypes.byref(_fargs(num_tokens=0, workspace=None)), None) == binding.OK
