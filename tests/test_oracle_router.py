"""Pins of the router-backward oracle (page 3, sonic-moe functional/backward.py:
the softmax-over-top-k, top-k-over-softmax and top-k scatter backward kernels).

The oracle's closed forms are checked against things other than themselves:
central finite differences of the forward maps (which are the plain
definitions), Jacobians assembled entry by entry, the shift invariance of the
softmax, and special cases with known answers."""
import numpy as np
import pytest

from oracle import router as R

MODES = [(R.SOFTMAX_OVER_TOPK, False), (R.TOPK_OVER_SOFTMAX, False), (R.TOPK_OVER_SOFTMAX, True), (R.TOPK, False)]


def _problem(T, E, K, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, scale, (T, E))
    idx = np.argsort(-z, axis=1, kind="stable")[:, :K]      # the top-k of each row
    g = rng.normal(0.0, 1.0, (T, K))
    return z, idx, g


@pytest.mark.parametrize("mode,renorm", MODES)
@pytest.mark.parametrize("T,E,K", [(5, 8, 2), (4, 7, 3), (3, 16, 8), (2, 5, 5)])
def test_backward_matches_finite_differences(mode, renorm, T, E, K):
    z, idx, g = _problem(T, E, K, seed=E * 10 + K)
    got = R.backward(mode, z, idx, g, renorm)
    h = 1e-6
    fd = np.zeros_like(z)
    for t in range(T):
        for j in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, j] += h
            zm[t, j] -= h
            fd[t, j] = ((g * R.forward(mode, zp, idx, renorm)).sum() - (g * R.forward(mode, zm, idx, renorm)).sum()) / (2 * h)
    assert np.max(np.abs(got - fd)) <= 1e-7 * max(1.0, np.max(np.abs(fd)))


@pytest.mark.parametrize("mode,renorm", MODES)
def test_closed_form_equals_assembled_jacobian(mode, renorm):
    z, idx, g = _problem(6, 9, 4, seed=3)
    a = R.backward(mode, z, idx, g, renorm)
    b = R.backward_jacobian(mode, z, idx, g, renorm)
    assert np.max(np.abs(a - b)) <= 1e-13


@pytest.mark.parametrize("mode,renorm", MODES[:3])
def test_softmax_modes_are_shift_invariant(mode, renorm):
    """softmax(z + c) = softmax(z): the gradient sums to zero over each row and
    does not change when a constant is added to a row's logits."""
    z, idx, g = _problem(7, 12, 3, seed=5)
    d = R.backward(mode, z, idx, g, renorm)
    assert np.max(np.abs(d.sum(axis=1))) <= 1e-14 * max(1.0, np.abs(d).max())
    d2 = R.backward(mode, z + np.arange(7)[:, None] * 3.5, idx, g, renorm)
    assert np.max(np.abs(d - d2)) <= 1e-13


def test_all_experts_selected_makes_the_softmax_modes_agree():
    """With K = E every mode over a softmax is the full softmax: the three
    softmax variants give the same gradient."""
    z, idx, g = _problem(4, 6, 6, seed=11)
    a = R.backward(R.SOFTMAX_OVER_TOPK, z, idx, g)
    b = R.backward(R.TOPK_OVER_SOFTMAX, z, idx, g, False)
    c = R.backward(R.TOPK_OVER_SOFTMAX, z, idx, g, True)
    assert np.max(np.abs(a - b)) <= 1e-14 and np.max(np.abs(a - c)) <= 1e-14


def test_single_expert_softmax_scores_are_constant():
    """K = 1: softmax over one logit and a renormalised single probability are
    both identically 1, so no gradient reaches the logits."""
    z, idx, g = _problem(5, 8, 1, seed=2)
    assert not R.backward(R.SOFTMAX_OVER_TOPK, z, idx, g).any()
    assert np.max(np.abs(R.backward(R.TOPK_OVER_SOFTMAX, z, idx, g, True))) <= 1e-16


def test_topk_scatter_and_unselected_zeros():
    z, idx, g = _problem(6, 10, 3, seed=4)
    d = R.backward(R.TOPK, z, idx, g)
    for t in range(6):
        for j in range(10):
            hit = np.nonzero(idx[t] == j)[0]
            assert d[t, j] == (g[t, hit[0]] if hit.size else 0.0)
    # softmax over the top-k also leaves the unselected logits without gradient,
    # top-k over the softmax does not
    s = R.backward(R.SOFTMAX_OVER_TOPK, z, idx, g)
    f = R.backward(R.TOPK_OVER_SOFTMAX, z, idx, g)
    mask = np.ones_like(z, dtype=bool)
    np.put_along_axis(mask, idx, False, axis=1)
    assert not s[mask].any() and np.all(f[mask] != 0)


def test_given_scores_equal_recomputed_ones():
    z, idx, g = _problem(5, 9, 3, seed=8)
    for mode, renorm in MODES[:3]:
        s = R.forward(mode, z, idx, renorm)
        assert np.array_equal(R.backward(mode, z, idx, g, renorm, scores=s), R.backward(mode, z, idx, g, renorm))


def test_gather_scores_reads_the_masked_layout():
    daff = np.arange(4 * 6, dtype=np.float64).reshape(4, 6)
    idx = np.array([[5, 0], [1, 2], [3, 4], [0, 5]])
    assert np.array_equal(R.gather_scores(daff, idx), [[5, 0], [7, 8], [15, 16], [18, 23]])
