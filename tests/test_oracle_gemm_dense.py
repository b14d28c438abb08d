"""Pins of the oracle's MX GEMM emulation and of the dense backward (P2).

Against: numpy float64 matmuls of operands dequantised through torch's float8
dtypes, exact integer GEMMs (closed form), and lossless inputs whose MXFP8
backward must equal the exact backward.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import rel_fro

F8 = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def _deq_torch(codes, scales, fmt):
    v = torch.from_numpy(codes).view(F8[fmt]).to(torch.float64).numpy()
    return v * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def _bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_mx_gemm_equals_fp64_matmul_of_dequantised(fa, fb):
    rng = np.random.default_rng(10)
    M, N, K = 40, 24, 128
    a, b = _bits(rng.standard_normal((M, K))), _bits(rng.standard_normal((N, K)) * 0.02)
    ac, asc = oracle.quantize(a, 1, fa)
    bc, bsc = oracle.quantize(b, 1, fb)
    got = oracle.mx_gemm_nt(ac, asc, fa, bc, bsc, fb)
    ref = (_deq_torch(ac, asc, fa) @ _deq_torch(bc, bsc, fb).T).astype(np.float32)
    np.testing.assert_allclose(got, ref, rtol=2e-7, atol=0)


def test_mx_gemm_integer_closed_form():
    """Unit scales and codes of small integers: the product is an exact integer GEMM."""
    rng = np.random.default_rng(11)
    M, N, K = 16, 12, 96
    vals = np.arange(-8, 9)
    enc = {v: oracle.fp8_encode(float(v), oracle.E4M3) for v in vals}
    ia, ib = rng.choice(vals, (M, K)), rng.choice(vals, (N, K))
    ac = np.vectorize(enc.get)(ia).astype(np.uint8)
    bc = np.vectorize(enc.get)(ib).astype(np.uint8)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    got = oracle.mx_gemm_nt(ac, ones_a, 0, bc, ones_b, 0)
    assert np.array_equal(got, (ia @ ib.T).astype(np.float32))


def test_dense_lossless_equals_exact():
    """Small-integer inputs survive both formats' quantisation losslessly, so the
    MXFP8 backward equals dX = dY W and dW = dY^T X exactly (then one bf16 rounding)."""
    rng = np.random.default_rng(12)
    M, N, K = 64, 96, 80
    dy, w, x = (rng.integers(-8, 9, s).astype(np.float32) for s in ((M, N), (N, K), (M, K)))
    dX, dW = oracle.dense_bwd(_bits(dy), _bits(w), _bits(x))
    ref_dx = _bits((dy.astype(np.int64) @ w.astype(np.int64)).astype(np.float32))
    ref_dw = _bits((dy.astype(np.int64).T @ x.astype(np.int64)).astype(np.float32))
    assert np.array_equal(dX, ref_dx) and np.array_equal(dW, ref_dw)


def test_dense_equals_composition_of_quantise_and_gemm():
    """The contraction-axis reading: dX uses dY and W quantised along N,
    dW uses dY and X quantised along M."""
    rng = np.random.default_rng(13)
    M, N, K = 64, 96, 64
    dy, w, x = _bits(rng.standard_normal((M, N))), _bits(rng.standard_normal((N, K)) * 0.02), \
        _bits(rng.standard_normal((M, K)))
    dX, dW = oracle.dense_bwd(dy, w, x)
    a, asc = oracle.quantize(dy, 1, oracle.E5M2)
    b, bsc = oracle.quantize(np.ascontiguousarray(w.T), 1, oracle.E4M3)
    ref = oracle.mx_gemm_nt(a, asc, 1, b, bsc, 0)
    assert np.array_equal(dX, _bits(ref))
    a, asc = oracle.quantize(np.ascontiguousarray(dy.T), 1, oracle.E5M2)
    b, bsc = oracle.quantize(np.ascontiguousarray(x.T), 1, oracle.E4M3)
    ref = oracle.mx_gemm_nt(a, asc, 1, b, bsc, 0)
    assert np.array_equal(dW, _bits(ref))


def test_dense_close_to_exact_and_row_selection():
    rng = np.random.default_rng(14)
    M, N, K = 96, 128, 64
    dy32, w32, x32 = rng.standard_normal((M, N)), rng.standard_normal((N, K)) * 0.02, rng.standard_normal((M, K))
    dy, w, x = _bits(dy32), _bits(w32), _bits(x32)
    bfv = lambda b: oracle.bf16_to_float(b).astype(np.float64)
    dX, dW = oracle.dense_bwd(dy, w, x)
    assert rel_fro(bfv(dX), bfv(dy) @ bfv(w)) < 0.08        # e5m2 x e4m3 noise, ~4-5%
    assert rel_fro(bfv(dW), bfv(dy).T @ bfv(x)) < 0.08
    assert rel_fro(bfv(dX), bfv(dy) @ bfv(w)) > 1e-3         # and it is not the exact product
    rows = np.array([5, 0, 77])
    sx, sw = oracle.dense_bwd(dy, w, x, dx_rows=rows, dw_rows=rows)
    assert np.array_equal(sx, dX[rows]) and np.array_equal(sw, dW[rows])


def test_dense_finite_differences_of_the_forward():
    """With quantisation switched off (format hook -1) the oracle's dX and dW are
    the gradients of L(X, W) = <dY, X W^T> ([P2] Background: Y = X W^T).  Central
    differences of L, evaluated by numpy's float64 matmul, must match every
    entry to one bf16 rounding; a transposed operand or a wrong contraction
    axis fails here."""
    rng = np.random.default_rng(14)
    M, N, K = 64, 32, 8
    dy, w, x = _bits(rng.standard_normal((M, N))), _bits(rng.standard_normal((N, K))), \
        _bits(rng.standard_normal((M, K)))
    dX, dW = oracle.dense_bwd(dy, w, x, fmt_dy=oracle.NONE, fmt_w=oracle.NONE, fmt_x=oracle.NONE)
    dyf, wf, xf = (oracle.bf16_to_float(v).astype(np.float64) for v in (dy, w, x))

    def loss(xv, wv):
        return float(np.sum(dyf * (xv @ wv.T)))

    h = 0.5
    fdx = np.zeros((M, K))
    for m in range(M):
        for k in range(K):
            xp, xm = xf.copy(), xf.copy()
            xp[m, k] += h
            xm[m, k] -= h
            fdx[m, k] = (loss(xp, wf) - loss(xm, wf)) / (2 * h)
    fdw = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            wp, wm = wf.copy(), wf.copy()
            wp[n, k] += h
            wm[n, k] -= h
            fdw[n, k] = (loss(xf, wp) - loss(xf, wm)) / (2 * h)
    gx = oracle.bf16_to_float(dX).astype(np.float64)
    gw = oracle.bf16_to_float(dW).astype(np.float64)
    assert np.all(np.abs(gx - fdx) <= 2.0 ** -8 * np.abs(fdx) + 1e-9)
    assert np.all(np.abs(gw - fdw) <= 2.0 ** -8 * np.abs(fdw) + 1e-9)
    assert np.abs(fdx).max() > 1 and np.abs(fdw).max() > 1
