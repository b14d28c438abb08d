"""Python binding of libmxfp8_moe.so (include/mxfp8_moe.h).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the library's gfx950 kernels.
There is no fallback -- if the shared library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

E4M3 = 0
E5M2 = 1
ACT_SWIGLU = 0
ACT_GEGLU = 1
ROUTER_SOFTMAX_OVER_TOPK = 0
ROUTER_TOPK_OVER_SOFTMAX = 1
ROUTER_TOPK = 2
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp8_moe.so")

_lib = None
_p = C.c_void_p
_i64 = C.c_int64


class MxError(RuntimeError):
    """A library call returned a non-zero mxfp8_status."""

    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed (status {status}): {msg}")
        self.status = status


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with mxfp8_grouped_gemm_amd/build.py "
                               "(or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


class MoeBwdArgs(C.Structure):
    _fields_ = [("T", _i64), ("H", _i64), ("I", _i64), ("E", _i64), ("N", _i64), ("block_size", _i64),
                ("hidden_states", _p), ("expert_affinities_masked", _p), ("gate_up_codes", _p),
                ("gate_up_scales", _p), ("down_codes", _p), ("down_scales", _p),
                ("token_position_to_id", _p), ("block_to_expert", _p), ("output_hidden_states_grad", _p),
                ("gate_up_proj_act_checkpoint_T", _p), ("down_proj_bias", _p),
                ("affinity_on", C.c_int), ("has_bias", C.c_int), ("fmt_weight", C.c_int),
                ("fmt_act", C.c_int), ("fmt_grad", C.c_int),
                ("hidden_states_grad", _p), ("expert_affinities_masked_grad", _p),
                ("gate_up_proj_weight_grad", _p), ("down_proj_weight_grad", _p),
                ("gate_and_up_proj_bias_grad", _p), ("down_proj_bias_grad", _p),
                ("gate_act_checkpoint_T", _p), ("intermediate_checkpoint_T", _p),
                ("scaled_intermediate_checkpoint_T", _p), ("down_proj_act_checkpoint", _p),
                ("num_valid_tokens", _p), ("accumulate", C.c_int), ("activation", C.c_int)]


LAYOUT_FIELDS = ("dy_codes", "dy_scales", "dy_deq", "wd_deq", "x_tok_codes", "x_tok_scales", "gy_tok_codes", "gy_tok_scales",
                 "inter_tok_codes", "inter_tok_scales", "dgu_row_codes", "dgu_row_scales", "dgu_tok_codes",
                 "dgu_tok_scales", "wgu_scales_pairs", "wd_scales_pairs", "phase1_ds", "phase1_tiles", "phase3_tiles", "dx_slot",
                 "phase3_parts", "slot_of", "daff_slot", "daff_part", "db1_acc", "db2_acc", "expert_block_offsets",
                 "expert_block_list", "slot_token", "slot_affinity", "block_flag", "total")


class MoeWorkspaceLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in LAYOUT_FIELDS]


def _declare(L):
    L.mxfp8_last_error.restype = C.c_char_p
    L.mxfp8_version.restype = C.c_char_p
    L.mxfp8_quantize.restype = C.c_int
    L.mxfp8_quantize.argtypes = [_p, _i64, _i64, C.c_int, C.c_int, _p, _p, _p]
    L.moe_num_blocks.restype = _i64
    L.moe_num_blocks.argtypes = [_i64, _i64, _i64, _i64]
    for name, res, args in (
        ("matmul_mxfp8_bwd_workspace_size", C.c_size_t, [_i64, _i64, _i64]),
        ("matmul_mxfp8_bwd_ex", C.c_int, [C.POINTER(MatmulBwdArgs), _p, C.c_size_t, _p]),
        ("matmul_mxfp8_bwd", C.c_int, [_p, _p, _p, _i64, _i64, _i64, C.c_int, C.c_int, C.c_int, _p, _p,
                                       _p, C.c_size_t, _p]),
        ("moe_build_blocks_workspace_size", C.c_size_t, [_i64]),
        ("moe_build_blocks", C.c_int, [_p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, C.c_size_t, _p]),
        ("moe_build_blocks_noalloc", C.c_int, [_p, _i64, _i64, _i64, _i64, _i64, _p, _p, _p]),
        ("moe_bwd_mxfp8_workspace_query", C.c_int, [C.POINTER(MoeBwdArgs), C.POINTER(MoeWorkspaceLayout)]),
        ("moe_bwd_mxfp8_workspace_size", C.c_size_t, [C.POINTER(MoeBwdArgs)]),
        ("moe_bwd_mxfp8", C.c_int, [C.POINTER(MoeBwdArgs), _p, C.c_size_t, _p]),
        ("moe_bwd_mxfp8_stage", C.c_int, [C.POINTER(MoeBwdArgs), _p, C.c_size_t, C.c_int, _p]),
        ("matmul_mxfp8_bwd_stage", C.c_int, [_p, _p, _p, _i64, _i64, _i64, C.c_int, C.c_int, C.c_int, _p, _p,
                                             _p, C.c_size_t, C.c_int, _p]),
        ("moe_router_bwd", C.c_int, [C.c_int, _i64, _i64, _i64, _p, _p, _p, _p, _p, C.c_int, _p, _p]),
    ):
        if hasattr(L, name):
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args


def version() -> str:
    return lib().mxfp8_version().decode()


def last_error() -> str:
    return lib().mxfp8_last_error().decode()


def _check(rc: int, name: str):
    if rc != 0:
        raise MxError(name, rc, last_error())


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: Optional[torch.Tensor], dtype, name):
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


# ----------------------------------------------------------------------------- quantiser
def mxfp8_quantize(x: torch.Tensor, axis: int = 1, fmt: int = E4M3, out=None):
    """x [rows, cols] bf16 -> (codes uint8 [rows, cols], scales uint8 E8M0).

    axis 1: groups of 32 along cols, scales [rows, cols/32];
    axis 0: groups of 32 along rows, scales [rows/32, cols].
    out: optional (codes, scales) of those shapes to write into."""
    rows, cols = x.shape
    sshape = (rows, cols // 32) if axis == 1 else (rows // 32, cols)
    if out is not None:
        codes, scales = out
        if tuple(codes.shape) != (rows, cols) or tuple(scales.shape) != sshape or \
                codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or \
                not codes.is_contiguous() or not scales.is_contiguous():
            raise ValueError("mxfp8_quantize: out must be contiguous uint8 tensors of the codes' and scales' shapes")
    else:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _check(lib().mxfp8_quantize(_dev(x, torch.bfloat16, "x"), rows, cols, axis, fmt, codes.data_ptr(),
                                scales.data_ptr(), _stream(x)), "mxfp8_quantize")
    return codes, scales


# ----------------------------------------------------------------------------- dense backward
def matmul_mxfp8_bwd(output_grad: torch.Tensor, weights: torch.Tensor, input_activation: torch.Tensor,
                     fmt_output_grad: int = E5M2, fmt_weights: int = E4M3, fmt_input: int = E4M3,
                     workspace: Optional[torch.Tensor] = None, out=None):
    """dX = dY W [M,K] and dW = dY^T X [N,K] for Y = X W^T (bf16 in, bf16 out)."""
    M, N = output_grad.shape
    K = weights.shape[1]
    L = lib()
    ws_bytes = L.matmul_mxfp8_bwd_workspace_size(M, N, K)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=output_grad.device)
    if out is None:
        out = (torch.empty((M, K), dtype=torch.bfloat16, device=output_grad.device),
               torch.empty((N, K), dtype=torch.bfloat16, device=output_grad.device))
    dx, dw = out
    _check(L.matmul_mxfp8_bwd(_dev(output_grad, torch.bfloat16, "output_grad"),
                              _dev(weights, torch.bfloat16, "weights"),
                              _dev(input_activation, torch.bfloat16, "input_activation"), M, N, K,
                              fmt_output_grad, fmt_weights, fmt_input, _dev(dx, torch.bfloat16, "dx"),
                              _dev(dw, torch.bfloat16, "dw"), workspace.data_ptr(), workspace.numel(),
                              _stream(output_grad)), "matmul_mxfp8_bwd")
    return dx, dw


class MatmulBwdArgs(C.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("output_grad", _p), ("weights", _p),
                ("input_activation", _p), ("fmt_output_grad", C.c_int), ("fmt_weights", C.c_int),
                ("fmt_input", C.c_int), ("output_grad_codes_n", _p), ("output_grad_scales_n", _p),
                ("output_grad_codes_m", _p), ("output_grad_scales_m", _p), ("weight_codes", _p),
                ("weight_scales", _p), ("input_codes", _p), ("input_scales", _p),
                ("output_grad_is_swizzled", C.c_int), ("weights_is_swizzled", C.c_int),
                ("input_is_swizzled", C.c_int), ("use_scale_packing", C.c_int), ("input_grad", _p),
                ("weight_grad", _p)]


def matmul_mxfp8_bwd_ex(M: int, N: int, K: int, device, output_grad=None, weights=None, input_activation=None,
                        fmt_output_grad: int = E5M2, fmt_weights: int = E4M3, fmt_input: int = E4M3,
                        output_grad_n=None, output_grad_m=None, weight_q=None, input_q=None,
                        output_grad_is_swizzled=False, weights_is_swizzled=False, input_is_swizzled=False,
                        use_scale_packing=False, workspace: Optional[torch.Tensor] = None, out=None):
    """matmul_mxfp8_bwd with [P2]'s optional pre-quantised operands
    (include/mxfp8_moe.h: matmul_mxfp8_bwd_ex).  output_grad_n / output_grad_m /
    weight_q / input_q are (codes uint8, scales uint8) pairs in the layouts the
    header gives, or None to quantise the bf16 tensor."""
    L = lib()
    if workspace is None:
        workspace = torch.empty(L.matmul_mxfp8_bwd_workspace_size(M, N, K), dtype=torch.uint8, device=device)
    if out is None:
        out = (torch.empty((M, K), dtype=torch.bfloat16, device=device),
               torch.empty((N, K), dtype=torch.bfloat16, device=device))
    dx, dw = out

    def q(pair, name):
        if pair is None:
            return None, None
        return _dev(pair[0], torch.uint8, name + " codes"), _dev(pair[1], torch.uint8, name + " scales")

    gn, gm, wq, xq = (q(output_grad_n, "output_grad_n"), q(output_grad_m, "output_grad_m"), q(weight_q, "weights"),
                      q(input_q, "input"))
    a = MatmulBwdArgs(M, N, K, _dev(output_grad, torch.bfloat16, "output_grad"), _dev(weights, torch.bfloat16, "weights"),
                      _dev(input_activation, torch.bfloat16, "input_activation"), fmt_output_grad, fmt_weights,
                      fmt_input, *gn, *gm, *wq, *xq, int(output_grad_is_swizzled), int(weights_is_swizzled),
                      int(input_is_swizzled), int(use_scale_packing), _dev(dx, torch.bfloat16, "dx"),
                      _dev(dw, torch.bfloat16, "dw"))
    _check(L.matmul_mxfp8_bwd_ex(C.byref(a), workspace.data_ptr(), workspace.numel(),
                                 C.c_void_p(torch.cuda.current_stream(torch.device(device)).cuda_stream)),
           "matmul_mxfp8_bwd_ex")
    return dx, dw


def matmul_mxfp8_bwd_stage(output_grad, weights, input_activation, stage: int, workspace, out,
                           fmt_output_grad: int = E5M2, fmt_weights: int = E4M3, fmt_input: int = E4M3):
    """One stage of matmul_mxfp8_bwd (0/1 quantise, 2 dX GEMM, 3 dW GEMM) on a filled workspace."""
    M, N = output_grad.shape
    K = weights.shape[1]
    dx, dw = out
    _check(lib().matmul_mxfp8_bwd_stage(output_grad.data_ptr(), weights.data_ptr(), input_activation.data_ptr(), M,
                                        N, K, fmt_output_grad, fmt_weights, fmt_input, dx.data_ptr(), dw.data_ptr(),
                                        workspace.data_ptr(), workspace.numel(), stage, _stream(output_grad)),
           "matmul_mxfp8_bwd_stage")


def matmul_workspace_regions(M: int, N: int, K: int):
    """Byte offsets of the dense workspace regions, as documented in the header."""
    def up(v):
        return (v + 255) // 256 * 256
    sizes = [(M * N, M * N // 32), (K * N, K * N // 32), (N * M, N * M // 32), (K * M, K * M // 32)]
    off, out = 0, []
    for c, s in sizes:
        co = off
        off = up(off + c)
        so = off
        off = up(off + s)
        out.append((co, so))
    return out


# ----------------------------------------------------------------------------- routing
def moe_num_blocks(T: int, K: int, E: int, block_size: int) -> int:
    return int(lib().moe_num_blocks(T, K, E, block_size))


def moe_build_blocks(topk_ids: torch.Tensor, E: int, block_size: int, N: Optional[int] = None, out=None,
                     workspace: Optional[torch.Tensor] = None):
    """topk_ids [T,K] int32 -> (token_position_to_id [N*B] int32, block_to_expert [N] int32)."""
    T, K = topk_ids.shape
    if N is None:
        N = moe_num_blocks(T, K, E, block_size)
    L = lib()
    ws = workspace if workspace is not None else torch.empty(L.moe_build_blocks_workspace_size(E),
                                                             dtype=torch.uint8, device=topk_ids.device)
    if out is None:
        out = (torch.empty(N * block_size, dtype=torch.int32, device=topk_ids.device),
               torch.empty(N, dtype=torch.int32, device=topk_ids.device))
    tpid, b2e = out
    _check(L.moe_build_blocks(_dev(topk_ids, torch.int32, "topk_ids"), T, K, E, block_size, N,
                              tpid.data_ptr(), b2e.data_ptr(), ws.data_ptr(), ws.numel(), _stream(topk_ids)),
           "moe_build_blocks")
    return tpid, b2e


def moe_build_blocks_noalloc(topk_ids: torch.Tensor, E: int, block_size: int, N: int, out):
    """moe_build_blocks through the allocation-free entry point: the caller
    passes the outputs (token_position_to_id [N*B], block_to_expert [N], int32),
    and neither the library nor this wrapper allocates device memory."""
    T, K = topk_ids.shape
    tpid, b2e = out
    for name, t, n in (("token_position_to_id", tpid, N * block_size), ("block_to_expert", b2e, N)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n or t.device != topk_ids.device:
            raise ValueError(f"{name}: need a contiguous int32 tensor of {n} entries on {topk_ids.device}")
    _check(lib().moe_build_blocks_noalloc(_dev(topk_ids, torch.int32, "topk_ids"), T, K, E, block_size, N,
                                          tpid.data_ptr(), b2e.data_ptr(), _stream(topk_ids)),
           "moe_build_blocks_noalloc")
    return tpid, b2e


# ----------------------------------------------------------------------------- MoE backward
class MoeBwd:
    """One MoE backward problem bound to device tensors (P1's argument list).

    Allocates the outputs and the workspace once; ``run()`` enqueues the whole
    backward on the current stream.  With ``accumulate=True`` the outputs are
    allocated zeroed and each ``run()`` adds its gradients into what they hold
    (write priors into ``self.out`` to start from other values)."""

    def __init__(self, hidden_states, expert_affinities_masked, gate_up_codes, gate_up_scales, down_codes,
                 down_scales, token_position_to_id, block_to_expert, output_hidden_states_grad, block_size,
                 gate_up_proj_act_checkpoint_T, down_proj_bias=None, affinity_on=0, fmt_weight=E4M3,
                 fmt_act=E4M3, fmt_grad=E5M2, workspace=None, gate_act_checkpoint_T=None,
                 intermediate_checkpoint_T=None, scaled_intermediate_checkpoint_T=None,
                 down_proj_act_checkpoint=None, num_valid_tokens=None, accumulate=False, activation=0):
        T, H = hidden_states.shape
        E, _, _, I = gate_up_codes.shape
        N = block_to_expert.numel()
        dev = hidden_states.device
        self.keep = [hidden_states, expert_affinities_masked, gate_up_codes, gate_up_scales, down_codes,
                     down_scales, token_position_to_id, block_to_expert, output_hidden_states_grad,
                     gate_up_proj_act_checkpoint_T, down_proj_bias, gate_act_checkpoint_T, intermediate_checkpoint_T,
                     scaled_intermediate_checkpoint_T, down_proj_act_checkpoint, num_valid_tokens]
        has_bias = down_proj_bias is not None
        alloc = torch.zeros if accumulate else torch.empty
        self.out = dict(
            dx=alloc((T, H), dtype=torch.bfloat16, device=dev),
            daff=alloc(T * E, dtype=torch.bfloat16, device=dev),
            dwgu=alloc((E, H, 2, I), dtype=torch.bfloat16, device=dev),
            dwd=alloc((E, I, H), dtype=torch.bfloat16, device=dev),
            db1=alloc((E, 2, I), dtype=torch.bfloat16, device=dev) if has_bias else None,
            db2=alloc((E, H), dtype=torch.bfloat16, device=dev) if has_bias else None)
        o = self.out
        self.args = MoeBwdArgs(
            T, H, I, E, N, block_size,
            _dev(hidden_states, torch.bfloat16, "hidden_states"),
            _dev(expert_affinities_masked, torch.float32, "expert_affinities_masked"),
            _dev(gate_up_codes, torch.uint8, "gate_up_codes"), _dev(gate_up_scales, torch.uint8, "gate_up_scales"),
            _dev(down_codes, torch.uint8, "down_codes"), _dev(down_scales, torch.uint8, "down_scales"),
            _dev(token_position_to_id, torch.int32, "token_position_to_id"),
            _dev(block_to_expert, torch.int32, "block_to_expert"),
            _dev(output_hidden_states_grad, torch.bfloat16, "output_hidden_states_grad"),
            _dev(gate_up_proj_act_checkpoint_T, torch.bfloat16, "gate_up_proj_act_checkpoint_T"),
            _dev(down_proj_bias, torch.bfloat16, "down_proj_bias"),
            affinity_on, int(has_bias), fmt_weight, fmt_act, fmt_grad,
            o["dx"].data_ptr(), o["daff"].data_ptr(), o["dwgu"].data_ptr(), o["dwd"].data_ptr(),
            o["db1"].data_ptr() if has_bias else None, o["db2"].data_ptr() if has_bias else None,
            _dev(gate_act_checkpoint_T, torch.bfloat16, "gate_act_checkpoint_T"),
            _dev(intermediate_checkpoint_T, torch.bfloat16, "intermediate_checkpoint_T"),
            _dev(scaled_intermediate_checkpoint_T, torch.bfloat16, "scaled_intermediate_checkpoint_T"),
            _dev(down_proj_act_checkpoint, torch.bfloat16, "down_proj_act_checkpoint"),
            _dev(num_valid_tokens, torch.int32, "num_valid_tokens"), int(bool(accumulate)), int(activation))
        L = lib()
        lay = MoeWorkspaceLayout()
        _check(L.moe_bwd_mxfp8_workspace_query(C.byref(self.args), C.byref(lay)), "moe_bwd_mxfp8_workspace_query")
        self.layout = {n: getattr(lay, n) for n in LAYOUT_FIELDS}
        if workspace is None:
            workspace = torch.empty(self.layout["total"], dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self.device = dev

    def run(self):
        _check(lib().moe_bwd_mxfp8(C.byref(self.args), self.workspace.data_ptr(), self.workspace.numel(),
                                   C.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)),
               "moe_bwd_mxfp8")
        return self.out

    NUM_STAGES = 10
    STAGE_NAMES = ("setup", "quantize_dy", "gather_quantize_x_dy", "bias", "phase1", "phase1_epilogue", "phase3",
                   "phase2", "phase4", "finalize")

    def stage(self, s: int):
        """Re-run one stage on the workspace a full run filled (profiling aid)."""
        _check(lib().moe_bwd_mxfp8_stage(C.byref(self.args), self.workspace.data_ptr(), self.workspace.numel(), s,
                                         C.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)),
               "moe_bwd_mxfp8_stage")

    def region(self, name: str, nbytes: int) -> torch.Tensor:
        """A uint8 view of one workspace region (for reading quantised operands back)."""
        off = self.layout[name]
        return self.workspace[off:off + nbytes]


def moe_bwd_mxfp8(*args, **kw):
    """Functional form: builds a MoeBwd and runs it once; returns the gradient dict."""
    return MoeBwd(*args, **kw).run()


# ----------------------------------------------------------------------------- router backward
def moe_router_bwd(mode: int, topk_idx: torch.Tensor, *, dscores: Optional[torch.Tensor] = None,
                   daff: Optional[torch.Tensor] = None, topk_scores: Optional[torch.Tensor] = None,
                   logits: Optional[torch.Tensor] = None, num_experts: Optional[int] = None, renorm: bool = False,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the router logits, [T, E] fp32 (include/mxfp8_moe.h: moe_router_bwd).

    topk_idx [T, K] int32; the upstream score gradients come either as dscores
    [T, K] fp32 or as daff, the bf16 affinity gradient in the masked layout
    ([T*E] or [T, E], as moe_bwd_mxfp8 returns it).  topk_scores [T, K] fp32 and
    logits [T, E] fp32 as the mode requires."""
    T, K = topk_idx.shape
    if num_experts is not None:
        E = int(num_experts)
    elif logits is not None:
        E = logits.shape[1]
    elif daff is not None:
        E = daff.numel() // max(T, 1)
    else:
        raise ValueError("moe_router_bwd: give num_experts (or logits / daff)")
    dev = topk_idx.device
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=dev)
    _check(lib().moe_router_bwd(mode, T, E, K, _dev(topk_idx, torch.int32, "topk_idx"),
                                _dev(topk_scores, torch.float32, "topk_scores"), _dev(logits, torch.float32, "logits"),
                                _dev(dscores, torch.float32, "dscores"), _dev(daff, torch.bfloat16, "daff"),
                                1 if renorm else 0, _dev(out, torch.float32, "out"), _stream(topk_idx)),
           "moe_router_bwd")
    return out
