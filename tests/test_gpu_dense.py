"""matmul_mxfp8_bwd on the GPU against the oracle (P2's dX = dY W, dW = dY^T X).

Bar: quantised operands in the workspace bit-exact; dX and dW within relative
Frobenius error 2e-3 (fp32 accumulation vs the oracle's exact sums, both then
rounded to bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import assert_parity, bf, pairs_to_rows, parity_stats, rel_fro, stage_major_to_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _mx():
    import mxfp8_grouped_gemm_amd as mx
    return mx


def _inputs(M, N, K, seed):
    cfg = S.DenseConfig("t", M, N, K, seed=seed)
    return S.dense_tensors(cfg, "cuda")


# N % 512 == 0 with M % 32 == 0 takes the one-pass dual-axis dY quantiser: M a
# multiple of 128 (pair-major dY^T scales) or not, and a partial last row tile
@pytest.mark.parametrize("M,N,K", [(64, 96, 128), (256, 320, 192), (96, 160, 544), (512, 384, 640),
                                   (32, 32, 32), (288, 544, 96), (256, 1024, 96), (96, 512, 160),
                                   (160, 512, 64), (640, 512, 416)])
def test_dense_small_full_parity(M, N, K):
    mx = _mx()
    t = _inputs(M, N, K, seed=M + N + K)
    ws = torch.zeros(mx.lib().matmul_mxfp8_bwd_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
    dx, dw = mx.matmul_mxfp8_bwd(t["dy"], t["w"], t["x"], workspace=ws)
    torch.cuda.synchronize()
    dy_b, w_b, x_b = (S.bf16_bits(t[k]) for k in ("dy", "w", "x"))
    rdx, rdw = oracle.dense_bwd(dy_b, w_b, x_b)
    sx = parity_stats(bf(S.bf16_bits(dx)), bf(rdx), rows=M)
    sw = parity_stats(bf(S.bf16_bits(dw)), bf(rdw), rows=N)
    print((M, N, K), "dX", sx, "dW", sw, flush=True)
    assert_parity("dX", sx, tol=TOL)
    assert_parity("dW", sw, tol=TOL)
    # quantised operands in the documented workspace regions, bit-exact
    regs = mx.matmul_workspace_regions(M, N, K)
    wsh = ws.cpu().numpy()
    want = [oracle.quantize(dy_b, 1, oracle.E5M2),
            oracle.quantize(np.ascontiguousarray(w_b.T), 1, oracle.E4M3),
            oracle.quantize(np.ascontiguousarray(dy_b.T), 1, oracle.E5M2),
            oracle.quantize(np.ascontiguousarray(x_b.T), 1, oracle.E4M3)]
    # scales of a GEMM whose contraction (N for [0],[1], M for [2],[3]) is a
    # multiple of 128 are stored pair-major, and its codes (both operands
    # quantised here from bf16) stage-major
    kdim = [N, N, M, M]
    for (co, so), (c, s), kk in zip(regs, want, kdim):
        got = wsh[co:co + c.size]
        if kk % 128 == 0:
            got = stage_major_to_rows(got, c.shape[0], kk)
        assert np.array_equal(got.ravel(), c.ravel())
        got = wsh[so:so + s.size]
        if kk % 128 == 0:
            got = pairs_to_rows(got, s.shape[0], kk)
        assert np.array_equal(got.ravel(), s.ravel())


@pytest.mark.parametrize("fdy,fw,fx", [(0, 0, 0), (1, 1, 1), (0, 1, 1), (1, 0, 1)])
def test_dense_format_combinations(fdy, fw, fx):
    mx = _mx()
    M, N, K = 192, 512, 320
    t = _inputs(M, N, K, seed=3)
    dx, dw = mx.matmul_mxfp8_bwd(t["dy"], t["w"], t["x"], fdy, fw, fx)
    rdx, rdw = oracle.dense_bwd(*(S.bf16_bits(t[k]) for k in ("dy", "w", "x")), fmt_dy=fdy, fmt_w=fw, fmt_x=fx)
    assert_parity("dX", parity_stats(bf(S.bf16_bits(dx)), bf(rdx), rows=M), tol=TOL)
    assert_parity("dW", parity_stats(bf(S.bf16_bits(dw)), bf(rdw), rows=N), tol=TOL)


def test_dense_4096_sampled_rows():
    """The benchmark's shape and launch configuration; the oracle computes a
    sample of output rows (each row spans every column tile)."""
    mx = _mx()
    cfg = S.DENSE
    t = S.dense_tensors(cfg, "cuda")
    dx, dw = mx.matmul_mxfp8_bwd(t["dy"], t["w"], t["x"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 255, 256, 4095], rng.integers(0, 4096, 28)]))
    rdx, rdw = oracle.dense_bwd(*(S.bf16_bits(t[k]) for k in ("dy", "w", "x")), dx_rows=rows, dw_rows=rows)
    gdx = bf(S.bf16_bits(dx))[rows]
    gdw = bf(S.bf16_bits(dw))[rows]
    sx = parity_stats(gdx, bf(rdx), rows=len(rows))
    sw = parity_stats(gdw, bf(rdw), rows=len(rows))
    print("dense 4096 sampled rows: dX", sx, "dW", sw, flush=True)
    assert_parity("dX", sx, tol=TOL)
    assert_parity("dW", sw, tol=TOL)
    # every output finite and not identically zero
    assert torch.isfinite(dx.float()).all() and torch.isfinite(dw.float()).all()
    assert dx.float().abs().sum() > 0 and dw.float().abs().sum() > 0


def test_dense_rejects_bad_shapes():
    mx = _mx()
    t = _inputs(64, 64, 64, 1)
    with pytest.raises(mx.MxError):
        mx.matmul_mxfp8_bwd(t["dy"][:, :48].contiguous(), t["w"][:48].contiguous(), t["x"])


def _prequantised(dy_b, w_b, x_b, swizzled, packed):
    """[P2]'s pre-quantised operands, made by the oracle's quantiser, in the
    layouts of matmul_mxfp8_bwd_ex: natural (as mxfp8_quantize writes them) or
    swizzled (contraction contiguous), scales row-major or packed pair-major."""
    from helpers import rows_to_pairs
    T = lambda a: np.ascontiguousarray(a.T)
    if not swizzled:
        ops = {"output_grad_n": oracle.quantize(dy_b, 1, oracle.E5M2),
               "output_grad_m": oracle.quantize(dy_b, 0, oracle.E5M2),
               "weight_q": oracle.quantize(w_b, 0, oracle.E4M3), "input_q": oracle.quantize(x_b, 0, oracle.E4M3)}
    else:
        ops = {"output_grad_n": oracle.quantize(dy_b, 1, oracle.E5M2),
               "output_grad_m": oracle.quantize(T(dy_b), 1, oracle.E5M2),
               "weight_q": oracle.quantize(T(w_b), 1, oracle.E4M3), "input_q": oracle.quantize(T(x_b), 1, oracle.E4M3)}
        if packed:
            ops = {k: (c, rows_to_pairs(s, c.shape[0], c.shape[1])) for k, (c, s) in ops.items()}
    return {k: (torch.from_numpy(np.ascontiguousarray(c)).cuda(), torch.from_numpy(np.ascontiguousarray(s)).cuda())
            for k, (c, s) in ops.items()}


@pytest.mark.parametrize("M,N,K,swizzled,packed", [(256, 320, 192, False, False), (512, 384, 640, False, False),
                                                   (96, 160, 544, False, False), (256, 320, 192, True, False),
                                                   (512, 384, 640, True, False), (512, 384, 640, True, True),
                                                   (96, 160, 544, True, False)])
def test_dense_prequantised_operands(M, N, K, swizzled, packed):
    """P2's pre-computed scales (codes + E8M0 scales per operand, dY once per
    contraction axis), unswizzled or in the GEMM's layout, row-major or packed
    scales: the outputs equal the bf16-input call bit for bit (the GEMMs read
    the same operand bytes) and keep parity with the oracle."""
    mx = _mx()
    t = _inputs(M, N, K, seed=M + 7 * N + K)
    dy_b, w_b, x_b = (S.bf16_bits(t[k]) for k in ("dy", "w", "x"))
    ref_dx, ref_dw = mx.matmul_mxfp8_bwd(t["dy"], t["w"], t["x"])
    ops = _prequantised(dy_b, w_b, x_b, swizzled, packed)
    flags = dict(output_grad_is_swizzled=swizzled, weights_is_swizzled=swizzled, input_is_swizzled=swizzled,
                 use_scale_packing=packed)
    # every operand pre-quantised: no bf16 input at all
    dx, dw = mx.matmul_mxfp8_bwd_ex(M, N, K, "cuda", **ops, **flags)
    # some pre-quantised, the rest quantised from bf16
    dx2, dw2 = mx.matmul_mxfp8_bwd_ex(M, N, K, "cuda", output_grad=t["dy"], input_activation=t["x"],
                                      output_grad_n=ops["output_grad_n"], weight_q=ops["weight_q"],
                                      output_grad_is_swizzled=swizzled, weights_is_swizzled=swizzled,
                                      use_scale_packing=packed)
    torch.cuda.synchronize()
    for a, b in ((dx, ref_dx), (dw, ref_dw), (dx2, ref_dx), (dw2, ref_dw)):
        assert torch.equal(a, b)
    rdx, rdw = oracle.dense_bwd(dy_b, w_b, x_b)
    assert_parity("dX", parity_stats(bf(S.bf16_bits(dx)), bf(rdx), rows=M), tol=TOL)
    assert_parity("dW", parity_stats(bf(S.bf16_bits(dw)), bf(rdw), rows=N), tol=TOL)
