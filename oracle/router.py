"""Router backward oracle -- TEST INFRASTRUCTURE ONLY.

Plain numpy in fp64.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the GPU library never does.

What it follows: page 3 (sonic-moe, functional/backward.py), the router
backward that consumes the affinity gradient d(a): its softmax-over-top-k,
top-k-over-softmax (with or without renormalisation of the selected
probabilities) and plain top-k scatter kernels.  The pages give those kernels'
closed forms; here each mode is written as the forward map from the router
logits to the K scores of a token and the vector-Jacobian product of that map,
built from the softmax Jacobian diag(p) - p p^T, so that the tests can pin it by
finite differences of the forward.

Shapes (one row per token): logits [T, E], idx [T, K] int (distinct expert ids
in [0, E)), scores [T, K], g = d(score) [T, K]; the result d(logits) is [T, E].
Positions a mode gives no gradient are 0.
"""
from __future__ import annotations

import numpy as np

SOFTMAX_OVER_TOPK = 0   # scores = softmax over the K selected logits
TOPK_OVER_SOFTMAX = 1   # scores = the K selected entries of softmax over all E logits
TOPK = 2                # scores = the K selected logits themselves


def _softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def forward(mode: int, logits: np.ndarray, idx: np.ndarray, renorm: bool = False) -> np.ndarray:
    """Scores [T, K] of each token for router mode `mode` (fp64)."""
    z = np.asarray(logits, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    sel = np.take_along_axis(z, idx, axis=1)
    if mode == SOFTMAX_OVER_TOPK:
        return _softmax(sel)
    if mode == TOPK_OVER_SOFTMAX:
        ps = np.take_along_axis(_softmax(z), idx, axis=1)
        return ps / ps.sum(axis=1, keepdims=True) if renorm else ps
    if mode == TOPK:
        return sel
    raise ValueError(f"unknown router mode {mode}")


def backward(mode: int, logits: np.ndarray, idx: np.ndarray, g: np.ndarray, renorm: bool = False,
             scores: np.ndarray | None = None) -> np.ndarray:
    """d(logits) [T, E] for upstream score gradients g [T, K] (fp64).

    SOFTMAX_OVER_TOPK: with y = softmax(logits[idx]) (or the given forward
      scores), the selected positions get J_y g = y * (g - <g, y>) (J_y is the
      symmetric softmax Jacobian); all other positions get 0.
    TOPK_OVER_SOFTMAX: p = softmax(logits) over all E.  Without renorm the
      scores are p[idx], so d(p) is g scattered to idx; with renorm they are
      p[idx] / S, S = sum p[idx], so d(p)[idx] = (g - <g, scores>) / S.  Then
      d(logits) = J_p d(p) = p * (d(p) - <d(p), p>) over every position.
    TOPK: g scattered to the selected positions.
    """
    z = np.asarray(logits, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    g = np.asarray(g, dtype=np.float64)
    T, E = z.shape
    out = np.zeros((T, E), dtype=np.float64)
    rows = np.arange(T)[:, None]
    if mode == SOFTMAX_OVER_TOPK:
        y = forward(mode, z, idx) if scores is None else np.asarray(scores, dtype=np.float64)
        out[rows, idx] = y * (g - (g * y).sum(axis=1, keepdims=True))
        return out
    if mode == TOPK_OVER_SOFTMAX:
        p = _softmax(z)
        dp = np.zeros((T, E), dtype=np.float64)
        if renorm:
            s = forward(mode, z, idx, True) if scores is None else np.asarray(scores, dtype=np.float64)
            S = np.take_along_axis(p, idx, axis=1).sum(axis=1, keepdims=True)
            dp[rows, idx] = (g - (g * s).sum(axis=1, keepdims=True)) / S
        else:
            dp[rows, idx] = g
        return p * (dp - (dp * p).sum(axis=1, keepdims=True))
    if mode == TOPK:
        out[rows, idx] = g
        return out
    raise ValueError(f"unknown router mode {mode}")


def backward_jacobian(mode: int, logits: np.ndarray, idx: np.ndarray, g: np.ndarray,
                      renorm: bool = False) -> np.ndarray:
    """The same product formed from explicit per-token Jacobians (small E):
    d(logits)_t = J_t^T g_t with J_t[k, j] = d score_k / d logit_j, built entry
    by entry from d p_i / d z_j = p_i (delta_ij - p_j)."""
    z = np.asarray(logits, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    g = np.asarray(g, dtype=np.float64)
    T, E = z.shape
    K = idx.shape[1]
    out = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        J = np.zeros((K, E))
        if mode == SOFTMAX_OVER_TOPK:
            y = _softmax(z[t, idx[t]])
            for k in range(K):
                for m in range(K):
                    J[k, idx[t, m]] = y[k] * ((1.0 if k == m else 0.0) - y[m])
        elif mode == TOPK_OVER_SOFTMAX:
            p = _softmax(z[t])
            dp = np.array([[p[i] * ((1.0 if i == j else 0.0) - p[j]) for j in range(E)] for i in range(E)])
            if renorm:
                S = p[idx[t]].sum()
                for k in range(K):
                    for i in idx[t]:
                        # d (p_ik / S) / d p_i
                        dsi = ((1.0 if i == idx[t, k] else 0.0) / S) - p[idx[t, k]] / S ** 2
                        J[k] += dsi * dp[i]
            else:
                for k in range(K):
                    J[k] = dp[idx[t, k]]
        elif mode == TOPK:
            for k in range(K):
                J[k, idx[t, k]] = 1.0
        else:
            raise ValueError(f"unknown router mode {mode}")
        out[t] = J.T @ g[t]
    return out


def gather_scores(daff: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g [T, K] from an affinity gradient laid out [T, E] (the masked layout of
    the affinities, index t*E + e): g[t, k] = daff[t, idx[t, k]]."""
    return np.take_along_axis(np.asarray(daff, dtype=np.float64), np.asarray(idx, dtype=np.int64), axis=1)
