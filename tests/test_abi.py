"""The C ABI without a GPU: the library loads, exports every function that
include/*.h declares, and rejects bad arguments before touching the device."""
import ctypes as C
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"typedef\s+struct\s*\{.*?\}\s*\w+\s*;", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", src, flags=re.M):
            if m.group(1) not in ("if", "return"):
                names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    names = _declared()
    assert {"mxfp8_quantize", "matmul_mxfp8_bwd", "moe_bwd_mxfp8", "moe_build_blocks", "moe_router_bwd"} <= names
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing


def test_validation_without_gpu():
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    fake = C.c_void_p(0x10000)           # never dereferenced: validation fails first
    assert L.mxfp8_quantize(fake, 32, 48, 1, 0, fake, fake, None) == 1
    assert "32" in mx.last_error()
    assert L.mxfp8_quantize(fake, 32, 32, 1, 9, fake, fake, None) == 1
    assert L.mxfp8_quantize(None, 32, 32, 1, 0, fake, fake, None) == 1
    assert L.mxfp8_quantize(fake, 0, 0, 1, 0, None, None, None) == 0     # empty: nothing to do
    assert L.moe_num_blocks(256, 2, 4, 128) == 7
    assert L.moe_num_blocks(32768, 8, 128, 128) == 2175
    assert L.moe_num_blocks(2, 1, 4, 128) == -1
    assert mx.version().startswith("mxfp8_moe")
    # router backward: every bad argument is caught before any launch
    rb = L.moe_router_bwd
    assert rb(3, 4, 8, 2, fake, fake, fake, fake, None, 0, fake, None) == 1 and "mode" in mx.last_error()
    assert rb(0, 4, 8, 9, fake, fake, fake, fake, None, 0, fake, None) == 1              # K > E
    assert rb(0, 4, 64, 33, fake, fake, fake, fake, None, 0, fake, None) == 1           # K above the bound
    assert rb(0, 4, 8, 2, fake, fake, fake, fake, None, 1, fake, None) == 1 and "renorm" in mx.last_error()
    assert rb(2, 4, 8, 2, fake, None, None, fake, fake, 0, fake, None) == 1              # both gradients
    assert rb(2, 4, 8, 2, fake, None, None, None, None, 0, fake, None) == 1              # neither
    assert rb(0, 4, 8, 2, fake, None, None, fake, None, 0, fake, None) == 1              # scores missing
    assert rb(1, 4, 8, 2, fake, None, None, fake, None, 0, fake, None) == 1              # logits missing
    assert rb(2, 4, 8, 2, C.c_void_p(0x10004), None, None, fake, None, 0, fake, None) == 1 and "aligned" in mx.last_error()
    assert rb(2, 0, 8, 2, None, None, None, fake, None, 0, None, None) == 0             # no tokens


@pytest.mark.parametrize("cls,ctype", [("MoeBwdArgs", "moe_bwd_mxfp8_args"),
                                       ("MoeWorkspaceLayout", "moe_bwd_mxfp8_workspace_layout"),
                                       ("MatmulBwdArgs", "matmul_mxfp8_bwd_args")])
def test_binding_structs_match_the_header(cls, ctype, tmp_path):
    """The ctypes mirrors of the header's structs: same size and every field at
    the offset the C compiler gives it."""
    import subprocess
    import mxfp8_grouped_gemm_amd as mx
    S = getattr(mx, cls)
    lines = [f'printf("size %zu\\n", sizeof({ctype}));']
    lines += [f'printf("{n} %zu\\n", offsetof({ctype}, {n}));' for n, _ in S._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"mxfp8_moe.h\"\nint main(void) {\n"
                   + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                 text=True).stdout.splitlines())
    assert int(got.pop("size")) == C.sizeof(S)
    for n, _ in S._fields_:
        assert int(got[n]) == getattr(S, n).offset, n


def test_moe_bwd_rejects_a_bad_accumulate_flag_without_gpu():
    """The accumulation flag is 0 or 1; anything else fails in validation,
    before any device access (the pointers here are never dereferenced)."""
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    fake = 0x10000
    T, H, I, E, B = 256, 128, 256, 4, 128
    N = L.moe_num_blocks(T, 2, E, B)
    ptrs = [fake] * 10
    a = mx.MoeBwdArgs(T, H, I, E, N, B, *ptrs, None, 0, 0, mx.E4M3, mx.E4M3, mx.E5M2,
                      fake, fake, fake, fake, None, None, None, None, None, None, None, 2)
    assert L.moe_bwd_mxfp8(C.byref(a), C.c_void_p(fake), 1 << 40, None) == 1
    assert "accumulate" in mx.last_error()


def _fake_args(mx, L, T=256, H=128, I=256, E=4, B=128, accumulate=0, bias=False):
    fake = 0x10000
    N = L.moe_num_blocks(T, 2, E, B)
    a = mx.MoeBwdArgs(T, H, I, E, N, B, *([fake] * 10), None, 0, 0, mx.E4M3, mx.E4M3, mx.E5M2,
                      fake, fake, fake, fake, None, None, None, None, None, None, None, accumulate)
    if bias:
        a.has_bias = 1
        a.down_proj_bias = a.gate_and_up_proj_bias_grad = a.down_proj_bias_grad = fake
    return a


def test_moe_bwd_workspace_and_size_limits_without_gpu():
    """A workspace below the size query is MXFP8_ERR_WORKSPACE (3); T * H of
    2^31 or more, or a [T,H] bf16 tensor of 2 GiB or more with H not a multiple
    of 128, is MXFP8_ERR_UNSUPPORTED (2): all found in validation, before any
    device access (the pointers are never dereferenced)."""
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    a = _fake_args(mx, L)
    need = L.moe_bwd_mxfp8_workspace_size(C.byref(a))
    assert need > 0
    assert L.moe_bwd_mxfp8(C.byref(a), C.c_void_p(0x10000), need - 1, None) == 3
    assert "workspace" in mx.last_error()
    assert L.moe_bwd_mxfp8(C.byref(a), C.c_void_p(0x10000), 1024, None) == 3
    # T * H = 2^31: one past the limit; one token fewer is accepted by validation,
    # with or without a bias (4 GiB bf16 tensors)
    big = _fake_args(mx, L, T=524288, H=4096, I=256, E=8, B=1024)
    assert L.moe_bwd_mxfp8(C.byref(big), C.c_void_p(0x10000), 1 << 62, None) == 2
    assert "32-bit" in mx.last_error()
    assert L.moe_bwd_mxfp8_workspace_size(C.byref(big)) == 0
    for bias in (False, True):
        ok = _fake_args(mx, L, T=524287, H=4096, I=256, E=8, B=1024, bias=bias)
        assert L.moe_bwd_mxfp8_workspace_size(C.byref(ok)) > 0
    # H not a multiple of 128: the bf16 [T,H] tensors stay under 2 GiB
    odd = _fake_args(mx, L, T=262144, H=4096 + 32, I=256, E=8, B=1024)
    assert L.moe_bwd_mxfp8(C.byref(odd), C.c_void_p(0x10000), 1 << 62, None) == 2
    assert "128" in mx.last_error()
    odd_ok = _fake_args(mx, L, T=262143 * 4096 // (4096 + 32), H=4096 + 32, I=256, E=8, B=1024)
    assert L.moe_bwd_mxfp8_workspace_size(C.byref(odd_ok)) > 0
    # more than 2^24 slots: a 256-row panel of a stage-major operand over the slots
    # would pass 2^32 bytes
    many = _fake_args(mx, L, T=8_500_000, H=32, I=256, E=8, B=1024)
    assert L.moe_bwd_mxfp8(C.byref(many), C.c_void_p(0x10000), 1 << 62, None) == 2
    assert "2^24" in mx.last_error()


def test_noalloc_build_blocks_validation_without_gpu():
    """The allocation-free routing entry point refuses, before any device call,
    an expert count above its scratch (UNSUPPORTED), too few blocks, null
    pointers and non-positive sizes (INVALID_ARG)."""
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    fake = C.c_void_p(0x10000)
    f = L.moe_build_blocks_noalloc
    assert f(fake, 8192, 1, 4097, 128, 4200, fake, fake, None) == 2 and "4096" in mx.last_error()
    assert f(fake, 256, 2, 4, 128, 6, fake, fake, None) == 1 and "worst case" in mx.last_error()
    assert f(None, 256, 2, 4, 128, 7, fake, fake, None) == 1
    assert f(fake, 256, 2, 4, 128, 7, None, fake, None) == 1
    assert f(fake, 0, 2, 4, 128, 7, fake, fake, None) == 1


def test_moe_bwd_rejects_an_unknown_activation_without_gpu():
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    a = _fake_args(mx, L)
    a.activation = 2
    assert L.moe_bwd_mxfp8(C.byref(a), C.c_void_p(0x10000), 1 << 40, None) == 1
    assert "activation" in mx.last_error()


def test_matmul_bwd_ex_validation_without_gpu():
    """The pre-quantised dense entry point refuses, before any device call,
    codes without scales, packed scales on an unswizzled operand or with a
    contraction that is not a multiple of 128, a swizzle flag without the
    operand it applies to, a flag outside {0,1}, and a missing bf16 input."""
    import mxfp8_grouped_gemm_amd as mx
    L = mx.lib()
    f = 0x10000

    def args(**kw):
        a = mx.MatmulBwdArgs(256, 256, 128, f, f, f, mx.E5M2, mx.E4M3, mx.E4M3)
        a.input_grad = a.weight_grad = f
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    run = lambda a: L.matmul_mxfp8_bwd_ex(C.byref(a), C.c_void_p(f), 1 << 40, None)
    assert run(args(weight_codes=f)) == 1 and "together" in mx.last_error()
    assert run(args(weight_codes=f, weight_scales=f, use_scale_packing=1)) == 1 and "swizzled" in mx.last_error()
    assert run(args(M=96, output_grad_codes_m=f, output_grad_scales_m=f, output_grad_is_swizzled=1,
                    use_scale_packing=1)) == 1 and "128" in mx.last_error()
    assert run(args(weights_is_swizzled=1)) == 1 and "weights_is_swizzled" in mx.last_error()
    assert run(args(input_is_swizzled=2)) == 1
    assert run(args(use_scale_packing=1)) == 1
    assert run(args(weights=None)) == 1 and "null" in mx.last_error()
    assert run(args(weights=None, weight_codes=f, weight_scales=f, output_grad=None)) == 1
    # every operand pre-quantised: no bf16 pointer is needed; only the workspace check remains
    a = args(output_grad=None, weights=None, input_activation=None, output_grad_codes_n=f, output_grad_scales_n=f,
             output_grad_codes_m=f, output_grad_scales_m=f, weight_codes=f, weight_scales=f, input_codes=f,
             input_scales=f)
    assert L.matmul_mxfp8_bwd_ex(C.byref(a), C.c_void_p(f), 16, None) == 3


def test_quantize_out_must_match_the_outputs():
    """mxfp8_quantize(out=...) checks the given buffers before any library call."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    good = (torch.empty((64, 128), dtype=torch.uint8), torch.empty((64, 4), dtype=torch.uint8))
    for bad in ((good[0][:, :64], good[1]), (good[0], torch.empty((64, 4), dtype=torch.int32)),
                (good[0], torch.empty((2, 128), dtype=torch.uint8)), (good[0].t(), good[1])):
        with pytest.raises(ValueError):
            mx.mxfp8_quantize(x, 1, mx.E4M3, out=bad)
