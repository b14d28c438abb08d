"""Router backward on the GPU against the fp64 oracle (page 3, sonic-moe
functional/backward.py: softmax-over-top-k, top-k-over-softmax, top-k scatter).

The kernel evaluates in fp32 (exp from the device math library).  Its outputs
are differences such as y_k (g_k - sum_m g_m y_m), which cancel, so the error
scales with the terms, not with the result: the bar is, element by element,
|gpu - oracle| <= 2e-5 * G, with G the largest |upstream gradient| of the row
(divided by the selected probability mass S under renormalisation, where the
kernel's terms are (g - <g, s>) / S).  An fp32 emulation of the kernel's
arithmetic reaches 1e-7 * G but up to 1.3e-4 of the row's largest output.
Inputs: normal router logits, the top-k of each row, the forward scores from
the oracle's forward rounded to fp32, normal upstream gradients."""
import numpy as np
import pytest
import torch

from oracle import router as R

pytestmark = pytest.mark.gpu
TOL = 2e-5

MODES = [(R.SOFTMAX_OVER_TOPK, False), (R.TOPK_OVER_SOFTMAX, False), (R.TOPK_OVER_SOFTMAX, True), (R.TOPK, False)]


def _inputs(T, E, K, seed):
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, 2.0, (T, E)).astype(np.float32)
    idx = np.argsort(-z, axis=1, kind="stable")[:, :K].astype(np.int32)
    g = rng.normal(0.0, 1.0, (T, K)).astype(np.float32)
    return z, idx, g


def _close(got, ref, g, scale=None):
    """scale: per-row divisor of the term size (S under renormalisation)."""
    G = np.abs(np.asarray(g, dtype=np.float64)).max(axis=1, keepdims=True)
    if scale is not None:
        G = G / np.asarray(scale, dtype=np.float64).reshape(-1, 1)
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    bound = TOL * G + 1e-30
    assert np.all(err <= bound), float((err / bound).max())


def _run(mode, renorm, z, idx, g, daff=None):
    import mxfp8_grouped_gemm_amd as mx
    T, E = z.shape
    scores = R.forward(mode, z, idx, renorm).astype(np.float32) if mode != R.TOPK else None
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = mx.moe_router_bwd(mode, dev(idx), dscores=None if daff is not None else dev(g), daff=daff,
                            topk_scores=dev(scores) if mode == R.SOFTMAX_OVER_TOPK or renorm else None,
                            logits=dev(z) if mode == R.TOPK_OVER_SOFTMAX else None, num_experts=E, renorm=renorm)
    torch.cuda.synchronize()
    ref = R.backward(mode, z.astype(np.float64), idx, g.astype(np.float64), renorm,
                     scores=None if scores is None else scores.astype(np.float64))
    S = R.forward(R.TOPK_OVER_SOFTMAX, z, idx).sum(axis=1) if renorm else None
    return out.cpu().numpy(), ref, S


@pytest.mark.parametrize("mode,renorm", MODES)
@pytest.mark.parametrize("T,E,K", [(1000, 8, 2), (4096, 128, 8), (333, 64, 6), (257, 16, 4), (50, 300, 32),
                                   (7, 3, 1), (129, 33, 5), (100, 24, 3), (64, 200, 8), (20, 600, 16)])
def test_router_bwd_matches_oracle(mode, renorm, T, E, K):
    z, idx, g = _inputs(T, E, K, seed=T + E + K)
    got, ref, S = _run(mode, renorm, z, idx, g)
    print(f"mode {mode} renorm {renorm} T {T} E {E} K {K}", flush=True)
    _close(got, ref, g, S)
    if mode != R.TOPK_OVER_SOFTMAX:   # unselected logits get exactly zero
        mask = np.ones_like(z, dtype=bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert not got[mask].any()


@pytest.mark.parametrize("mode,renorm", MODES)
def test_router_bwd_fine_workload_size(mode, renorm):
    """The fine workload's router: 32768 tokens, 128 experts, top-8."""
    z, idx, g = _inputs(32768, 128, 8, seed=5)
    got, ref, S = _run(mode, renorm, z, idx, g)
    _close(got, ref, g, S)


@pytest.mark.parametrize("mode,renorm", MODES)
def test_router_bwd_reads_the_affinity_gradient_layout(mode, renorm):
    """daff in the masked [T, E] bf16 layout gives the same result as the
    gathered fp32 gradients."""
    T, E, K = 500, 16, 3
    z, idx, _ = _inputs(T, E, K, seed=9)
    rng = np.random.default_rng(10)
    daff32 = np.zeros((T, E), dtype=np.float32)
    np.put_along_axis(daff32, idx.astype(np.int64), rng.normal(0, 1, (T, K)).astype(np.float32), axis=1)
    daff = torch.from_numpy(daff32).to(torch.bfloat16).cuda()
    g = R.gather_scores(daff.float().cpu().numpy(), idx).astype(np.float32)   # the bf16 values, exactly
    got_a, ref, S = _run(mode, renorm, z, idx, g, daff=daff.reshape(-1))
    got_g, _, _ = _run(mode, renorm, z, idx, g)
    assert np.array_equal(got_a, got_g)
    _close(got_a, ref, g, S)


def test_router_bwd_skips_out_of_range_indices():
    import mxfp8_grouped_gemm_amd as mx
    idx = torch.tensor([[0, -1], [5, 2], [7, 8]], dtype=torch.int32, device="cuda")
    g = torch.tensor([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]], dtype=torch.float32, device="cuda")
    out = mx.moe_router_bwd(R.TOPK, idx, dscores=g, num_experts=8).cpu().numpy()
    ref = np.zeros((3, 8), dtype=np.float32)
    ref[0, 0], ref[1, 5], ref[1, 2], ref[2, 7] = 1.0, 3.0, 4.0, 5.0
    assert np.array_equal(out, ref)


def test_router_bwd_after_moe_backward():
    """The router backward on d(a) straight from moe_bwd_mxfp8 (tiny MoE
    config): reading the bf16 output in place equals the gathered values."""
    import mxfp8_grouped_gemm_amd as mx
    import synthetic as S
    from moe_gpu_common import gpu_problem
    cfg = S.TINY
    gp = gpu_problem(cfg)
    out = gp["op"].run()
    torch.cuda.synchronize()
    topk = np.ascontiguousarray(gp["topk"]).astype(np.int32)
    T, E, K = cfg.T, cfg.E, cfg.K
    daff = out["daff"]
    g = R.gather_scores(daff.float().reshape(T, E).cpu().numpy(), topk).astype(np.float32)
    rng = np.random.default_rng(0)
    z = rng.normal(0, 1, (T, E)).astype(np.float32)
    for mode, renorm in MODES:
        got_a, ref, mass = _run(mode, renorm, z, topk, g, daff=daff.reshape(-1))
        _close(got_a, ref, g, mass)
