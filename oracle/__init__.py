"""CPU oracle for the MXFP8 MoE backward -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper over ``liboracle.so`` (plain C++ in fp64, ``mxfp8_oracle.cpp``).
Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the GPU library never does.

Arrays are numpy: bf16 tensors travel as ``uint16`` bit patterns, codes and E8M0
scales as ``uint8``.  Every function returns freshly allocated outputs.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

E4M3 = 0
E5M2 = 1
NONE = -1  # test hook: quantisation disabled
SWIGLU, GEGLU = 0, 1  # gated activations

_lib = None


def lib():
    """The loaded oracle library: liboracle.so, or the file MXFP8_ORACLE_LIB
    names (the sanitizer build, loaded by the sanitizer pin's child process)."""
    global _lib
    if _lib is None:
        path = os.environ.get("MXFP8_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i64 = C.c_int64


def _declare(L):
    L.orc_fp8_decode.restype = C.c_double
    L.orc_fp8_decode.argtypes = [C.c_int, C.c_int]
    L.orc_fp8_encode.restype = C.c_int
    L.orc_fp8_encode.argtypes = [C.c_double, C.c_int]
    L.orc_fp8_encode_array.restype = C.c_int
    L.orc_fp8_encode_array.argtypes = [_p, _i64, C.c_int, _p]
    L.orc_fp8_emax.restype = C.c_int
    L.orc_fp8_emax.argtypes = [C.c_int]
    L.orc_double_to_bf16.restype = C.c_uint16
    L.orc_double_to_bf16.argtypes = [C.c_double]
    L.orc_bf16_to_double.restype = C.c_double
    L.orc_bf16_to_double.argtypes = [C.c_uint16]
    L.orc_quantize_group.restype = C.c_int
    L.orc_quantize_group.argtypes = [_p, C.c_int, C.c_int, _p, _p]
    L.orc_quantize.restype = C.c_int
    L.orc_quantize.argtypes = [_p, _i64, _i64, C.c_int, C.c_int, _p, _p]
    L.orc_mx_gemm_nt.restype = C.c_int
    L.orc_mx_gemm_nt.argtypes = [_p, _p, C.c_int, _p, _p, C.c_int, _i64, _i64, _i64, _p, C.c_int]
    L.orc_dense_bwd.restype = C.c_int
    L.orc_dense_bwd.argtypes = [_p, _p, _p, _i64, _i64, _i64, C.c_int, C.c_int, C.c_int,
                                _p, _i64, _p, _p, _i64, _p, C.c_int]
    L.orc_num_blocks.restype = _i64
    L.orc_num_blocks.argtypes = [_i64, _i64, _i64, _i64]
    L.orc_build_blocks.restype = C.c_int
    L.orc_build_blocks.argtypes = [_p, _i64, _i64, _i64, _i64, _i64, _p, _p]
    L.orc_moe_bwd.restype = C.c_int
    L.orc_moe_bwd.argtypes = [_p, _p, _p, _p, _p, _p, _p]
    L.orc_moe_token_rows.restype = C.c_int
    L.orc_moe_token_rows.argtypes = [_p, _p, _i64, _p, _p]
    L.orc_moe_expert_cols.restype = C.c_int
    L.orc_moe_expert_cols.argtypes = [_p, _i64, _p, _i64, _p, _p, _p, _p]
    L.orc_moe_block_detail.restype = C.c_int
    L.orc_moe_block_detail.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _p]
    L.orc_moe_token_operand.restype = C.c_int
    L.orc_moe_token_operand.argtypes = [_p, C.c_int, _p, _p]
    L.orc_moe_fwd_exact.restype = C.c_int
    L.orc_moe_fwd_exact.argtypes = [_p, _p, _p]
    L.orc_moe_bwd_exact.restype = C.c_int
    L.orc_moe_bwd_exact.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p]


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# --------------------------------------------------------------------------- codec
def fp8_decode(code: int, fmt: int) -> float:
    return lib().orc_fp8_decode(int(code), fmt)


def fp8_encode(y: float, fmt: int) -> int:
    return lib().orc_fp8_encode(float(y), fmt)


def fp8_encode_array(y: np.ndarray, fmt: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64).ravel()
    out = np.zeros(y.size, np.uint8)
    _check(lib().orc_fp8_encode_array(_ptr(y), y.size, fmt, _ptr(out)), "encode_array")
    return out


def fp8_emax(fmt: int) -> int:
    return lib().orc_fp8_emax(fmt)


def double_to_bf16(x: float) -> int:
    return lib().orc_double_to_bf16(float(x))


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_group(v, fmt: int):
    """Returns (scale_byte, codes[32] uint8, dequantised[32] float64)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    codes = np.zeros(v.size, np.uint8)
    deq = np.zeros(v.size, np.float64)
    s = lib().orc_quantize_group(_ptr(v), v.size, fmt, _ptr(codes), _ptr(deq))
    return s, codes, deq


def quantize(x_bits: np.ndarray, axis: int, fmt: int):
    """x [R][C] bf16 bits -> (codes [R][C] u8, scales [R][C/32] (axis 1) or [R/32][C] (axis 0))."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, Cc = x.shape
    codes = np.zeros((R, Cc), np.uint8)
    scales = np.zeros((R, Cc // 32) if axis == 1 else (R // 32, Cc), np.uint8)
    _check(lib().orc_quantize(_ptr(x), R, Cc, axis, fmt, _ptr(codes), _ptr(scales)), "quantize")
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, axis: int, fmt: int) -> np.ndarray:
    """Dequantised float64 values of an MX tensor (uses the oracle's decode)."""
    table = np.array([fp8_decode(c, fmt) for c in range(256)], np.float64)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    sc = np.repeat(sc, 32, axis=axis)
    return table[codes] * sc


def mx_gemm_nt(a_codes, a_scales, fmt_a, b_codes, b_scales, fmt_b, nthreads=0):
    M, K = a_codes.shape
    N = b_codes.shape[0]
    out = np.zeros((M, N), np.float32)
    args = [np.ascontiguousarray(v) for v in (a_codes, a_scales, b_codes, b_scales)]
    _check(lib().orc_mx_gemm_nt(_ptr(args[0]), _ptr(args[1]), fmt_a, _ptr(args[2]), _ptr(args[3]),
                                fmt_b, M, N, K, _ptr(out), nthreads), "mx_gemm_nt")
    return out


def dense_bwd(dY, W, X, fmt_dy=E5M2, fmt_w=E4M3, fmt_x=E4M3, dx_rows=None, dw_rows=None,
              want_dx=True, want_dw=True, nthreads=0):
    """P2 dense backward.  Returns (dX rows bf16 bits, dW rows bf16 bits)."""
    dY, W, X = (np.ascontiguousarray(v, dtype=np.uint16) for v in (dY, W, X))
    M, N = dY.shape
    K = W.shape[1]
    rx = None if dx_rows is None else np.ascontiguousarray(dx_rows, dtype=np.int64)
    rw = None if dw_rows is None else np.ascontiguousarray(dw_rows, dtype=np.int64)
    dX = np.zeros((M if rx is None else rx.size, K), np.uint16) if want_dx else None
    dW = np.zeros((N if rw is None else rw.size, K), np.uint16) if want_dw else None
    _check(lib().orc_dense_bwd(_ptr(dY), _ptr(W), _ptr(X), M, N, K, fmt_dy, fmt_w, fmt_x,
                               _ptr(rx), 0 if rx is None else rx.size, _ptr(dX),
                               _ptr(rw), 0 if rw is None else rw.size, _ptr(dW), nthreads),
           "dense_bwd")
    return dX, dW


# --------------------------------------------------------------------------- routing
def num_blocks(T, K, E, B) -> int:
    return int(lib().orc_num_blocks(T, K, E, B))


def build_blocks(topk: np.ndarray, E: int, B: int, N: Optional[int] = None):
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    T, K = topk.shape
    if N is None:
        N = num_blocks(T, K, E, B)
    tpid = np.zeros(N * B, np.int32)
    b2e = np.zeros(N, np.int32)
    _check(lib().orc_build_blocks(_ptr(topk), T, K, E, B, N, _ptr(tpid), _ptr(b2e)), "build_blocks")
    return tpid, b2e


# --------------------------------------------------------------------------- MoE (MX mode)
class _MoeProblem(C.Structure):
    _fields_ = [("T", _i64), ("H", _i64), ("I", _i64), ("E", _i64), ("N", _i64), ("B", _i64),
                ("hidden", _p), ("aff", _p), ("wgu_codes", _p), ("wgu_scales", _p),
                ("wd_codes", _p), ("wd_scales", _p), ("tpid", _p), ("b2e", _p), ("dy", _p),
                ("ckpt", _p), ("b2", _p), ("affinity_on", C.c_int), ("has_bias", C.c_int),
                ("fmt_w", C.c_int), ("fmt_act", C.c_int), ("fmt_grad", C.c_int),
                ("nthreads", C.c_int), ("accumulate", C.c_int), ("activation", C.c_int)]


@dataclass
class MoeProblem:
    """Host copy of one MoE backward problem (P1's argument list).

    hidden, dy: [T,H] bf16 bits; aff: [T*E] float32; wgu_codes [E,H,2,I] u8 with
    wgu_scales [E,H,2,I/32]; wd_codes [E,I,H] with wd_scales [E,I,H/32]; tpid [N*B]
    int32; b2e [N] int32; ckpt [N,2,I,B] bf16 bits; b2 [E,H] bf16 bits or None.
    """
    T: int
    H: int
    I: int
    E: int
    N: int
    B: int
    hidden: np.ndarray
    aff: np.ndarray
    wgu_codes: np.ndarray
    wgu_scales: np.ndarray
    wd_codes: np.ndarray
    wd_scales: np.ndarray
    tpid: np.ndarray
    b2e: np.ndarray
    dy: np.ndarray
    ckpt: np.ndarray
    b2: Optional[np.ndarray] = None
    affinity_on: int = 0
    has_bias: int = 0
    fmt_w: int = E4M3
    fmt_act: int = E4M3
    fmt_grad: int = E5M2
    nthreads: int = 0
    accumulate: int = 0      # P1's accumulation flag: outputs = bf16(prior + gradient)
    activation: int = 0      # 0 = SwiGLU, 1 = GeGLU (the erf form of GELU)

    def _struct(self):
        keep = {}
        for name, dt in (("hidden", np.uint16), ("aff", np.float32), ("wgu_codes", np.uint8),
                         ("wgu_scales", np.uint8), ("wd_codes", np.uint8), ("wd_scales", np.uint8),
                         ("tpid", np.int32), ("b2e", np.int32), ("dy", np.uint16),
                         ("ckpt", np.uint16), ("b2", np.uint16)):
            v = getattr(self, name)
            keep[name] = None if v is None else np.ascontiguousarray(v, dtype=dt)
        s = _MoeProblem(self.T, self.H, self.I, self.E, self.N, self.B,
                        *[_ptr(keep[k]) for k in ("hidden", "aff", "wgu_codes", "wgu_scales",
                                                  "wd_codes", "wd_scales", "tpid", "b2e", "dy",
                                                  "ckpt", "b2")],
                        self.affinity_on, self.has_bias, self.fmt_w, self.fmt_act, self.fmt_grad,
                        self.nthreads, self.accumulate, self.activation)
        return s, keep


def _outputs(shapes, prior):
    """bf16-bit output arrays: zeros, or copies of prior[name] (the values an
    accumulating backward adds to)."""
    return {k: (np.zeros(shp, np.uint16) if prior is None or prior.get(k) is None
                else np.array(prior[k], np.uint16, order="C").reshape(shp)) for k, shp in shapes.items()}


def moe_bwd(p: MoeProblem, prior=None):
    """Full MX-mode backward: dict of bf16-bit arrays dx, daff, dwgu, dwd, db1, db2.
    With p.accumulate, prior[name] holds the outputs' values on entry."""
    s, keep = p._struct()
    out = _outputs(dict(dx=(p.T, p.H), daff=(p.T * p.E,), dwgu=(p.E, p.H, 2, p.I), dwd=(p.E, p.I, p.H),
                        db1=(p.E, 2, p.I), db2=(p.E, p.H)), prior)
    _check(lib().orc_moe_bwd(C.byref(s), *[_ptr(out[k]) for k in ("dx", "daff", "dwgu", "dwd", "db1", "db2")]),
           "moe_bwd")
    del keep
    return out


def moe_token_rows(p: MoeProblem, tokens, prior=None):
    """dX rows and d(a) rows ([E] per token) of the given tokens; with
    p.accumulate, prior = dict(dx=[n,H], daff=[n,E]) of their values on entry."""
    s, keep = p._struct()
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    o = _outputs(dict(dx=(tok.size, p.H), daff=(tok.size, p.E)), prior)
    dx, da = o["dx"], o["daff"]
    _check(lib().orc_moe_token_rows(C.byref(s), _ptr(tok), tok.size, _ptr(dx), _ptr(da)), "token_rows")
    del keep
    return dx, da


def moe_expert_cols(p: MoeProblem, e: int, icols, prior=None):
    """Expert e's weight and bias gradients at intermediate columns icols; with
    p.accumulate, prior holds their values on entry (same shapes as returned)."""
    s, keep = p._struct()
    ic = np.ascontiguousarray(icols, dtype=np.int32)
    n = ic.size
    o = _outputs(dict(dwgu=(p.H, 2, n), dwd=(n, p.H), db1=(2, n), db2=(p.H,)), prior)
    dwgu, dwd, db1, db2 = o["dwgu"], o["dwd"], o["db1"], o["db2"]
    _check(lib().orc_moe_expert_cols(C.byref(s), e, _ptr(ic), n, _ptr(dwgu), _ptr(dwd), _ptr(db1),
                                     _ptr(db2)), "expert_cols")
    del keep
    return dict(dwgu=dwgu, dwd=dwd, db1=db1, db2=db2)


def moe_block_detail(p: MoeProblem, b: int):
    s, keep = p._struct()
    out = dict(dS=np.zeros((p.B, p.I), np.float32), ga=np.zeros((p.B, p.I), np.uint16),
               inter=np.zeros((p.B, p.I), np.uint16), dG=np.zeros((p.B, p.I), np.uint16),
               dU=np.zeros((p.B, p.I), np.uint16), daff_slot=np.zeros(p.B, np.float32))
    _check(lib().orc_moe_block_detail(C.byref(s), b, *[_ptr(out[k]) for k in
                                                       ("dS", "ga", "inter", "dG", "dU", "daff_slot")]),
           "block_detail")
    del keep
    return out


TOK_X, TOK_GY, TOK_INTER, TOK_DGU = 0, 1, 2, 3


def moe_token_operand(p: MoeProblem, which: int):
    """Token-axis quantised GEMM operand: (codes [rows][N*B], scales [rows][N*B/32])."""
    s, keep = p._struct()
    P = p.N * p.B
    rows = p.H if which <= 1 else (p.I if which == 2 else 2 * p.I)
    codes = np.zeros((rows, P), np.uint8)
    scales = np.zeros((rows, P // 32), np.uint8)
    _check(lib().orc_moe_token_operand(C.byref(s), which, _ptr(codes), _ptr(scales)), "token_operand")
    del keep
    return codes, scales


# --------------------------------------------------------------------------- MoE (exact mode)
class _MoeExact(C.Structure):
    _fields_ = [("T", _i64), ("H", _i64), ("I", _i64), ("E", _i64), ("N", _i64), ("B", _i64),
                ("x", _p), ("aff", _p), ("wgu", _p), ("b1", _p), ("wd", _p), ("b2", _p),
                ("tpid", _p), ("b2e", _p), ("affinity_on", C.c_int), ("activation", C.c_int)]


@dataclass
class MoeExact:
    """fp64 problem: x [T,H], aff [T*E], wgu [E,H,2,I], b1 [E,2,I]|None, wd [E,I,H], b2 [E,H]|None."""
    x: np.ndarray
    aff: np.ndarray
    wgu: np.ndarray
    wd: np.ndarray
    tpid: np.ndarray
    b2e: np.ndarray
    B: int
    b1: Optional[np.ndarray] = None
    b2: Optional[np.ndarray] = None
    affinity_on: int = 0
    activation: int = 0      # 0 = SwiGLU, 1 = GeGLU

    def _struct(self):
        T, H = self.x.shape
        E, _, _, I = self.wgu.shape
        N = self.b2e.size
        keep = {k: (None if getattr(self, k) is None else
                    np.ascontiguousarray(getattr(self, k), dtype=np.float64))
                for k in ("x", "aff", "wgu", "b1", "wd", "b2")}
        keep["tpid"] = np.ascontiguousarray(self.tpid, dtype=np.int32)
        keep["b2e"] = np.ascontiguousarray(self.b2e, dtype=np.int32)
        s = _MoeExact(T, H, I, E, N, self.B, *[_ptr(keep[k]) for k in
                                               ("x", "aff", "wgu", "b1", "wd", "b2", "tpid", "b2e")],
                      self.affinity_on, self.activation)
        return s, keep, (T, H, I, E, N)


def moe_fwd_exact(p: MoeExact, want_ckpt=False):
    s, keep, (T, H, I, E, N) = p._struct()
    y = np.zeros((T, H), np.float64)
    ck = np.zeros((N, 2, I, p.B), np.float64) if want_ckpt else None
    _check(lib().orc_moe_fwd_exact(C.byref(s), _ptr(y), _ptr(ck)), "fwd_exact")
    del keep
    return (y, ck) if want_ckpt else y


def moe_bwd_exact(p: MoeExact, dy: np.ndarray):
    s, keep, (T, H, I, E, N) = p._struct()
    dyc = np.ascontiguousarray(dy, dtype=np.float64)
    out = dict(dx=np.zeros((T, H)), daff=np.zeros(T * E), dwgu=np.zeros((E, H, 2, I)),
               dwd=np.zeros((E, I, H)), db1=np.zeros((E, 2, I)), db2=np.zeros((E, H)))
    _check(lib().orc_moe_bwd_exact(C.byref(s), _ptr(dyc), *[_ptr(out[k]) for k in
                                                          ("dx", "daff", "dwgu", "dwd", "db1", "db2")]),
           "bwd_exact")
    del keep
    return out
