"""Pins of the routing-block construction (P1: token_position_to_id,
block_to_expert and the block count N in the "Dimensions" paragraph)."""
import itertools

import numpy as np
import pytest

import oracle


def _compositions(total, parts):
    if parts == 1:
        yield (total,)
        return
    for first in range(total + 1):
        for rest in _compositions(total - first, parts - 1):
            yield (first,) + rest


def test_block_count_formula_is_worst_case():
    """N = (T*TopK - (E-1))/B + E - 1 with ceiling division equals the maximum of
    sum_e ceil(n_e/B) over every load vector with sum n_e = T*TopK."""
    for E in (1, 2, 3):
        for B in (1, 2, 3, 4):
            for TK in range(E, 10):
                worst = max(sum((n + B - 1) // B for n in c) for c in _compositions(TK, E))
                assert oracle.num_blocks(TK, 1, E, B) == worst, (E, B, TK)


def _reference_blocks(topk, E, B, N):
    """Brute force: stable sort of the (expert, token) pairs, then pad per expert."""
    pairs = sorted((int(e), t) for t in range(topk.shape[0]) for e in topk[t] if e >= 0)
    tp, be = [], []
    for e in range(E):
        toks = [t for (ee, t) in pairs if ee == e]
        nb = -(-len(toks) // B)
        tp += toks + [-1] * (nb * B - len(toks))
        be += [e] * nb
    tp += [-1] * (N * B - len(tp))
    be += [E - 1] * (N - len(be))
    return np.array(tp, np.int32), np.array(be, np.int32)


@pytest.mark.parametrize("T,K,E,B", [(40, 2, 4, 8), (64, 3, 7, 4), (100, 1, 3, 32), (33, 4, 16, 8)])
def test_build_blocks_bruteforce_and_invariants(T, K, E, B):
    rng = np.random.default_rng(T * 31 + E)
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    N = oracle.num_blocks(T, K, E, B)
    tpid, b2e = oracle.build_blocks(topk, E, B, N)
    rt, rb = _reference_blocks(topk, E, B, N)
    assert np.array_equal(tpid, rt) and np.array_equal(b2e, rb)
    # every routed pair exactly once, each block a single expert, experts contiguous
    seen = sorted((int(b2e[s // B]), int(tpid[s])) for s in range(N * B) if tpid[s] >= 0)
    assert seen == sorted((int(e), t) for t in range(T) for e in topk[t])
    assert np.all(np.diff(b2e) >= 0)


def test_build_blocks_rejects_small_N_and_bad_ids():
    topk = np.array([[0, 1], [1, 2]], np.int32)
    N = oracle.num_blocks(2, 2, 3, 4)
    with pytest.raises(ValueError):
        oracle.build_blocks(topk, 3, 4, 2)          # needs 3 blocks
    oracle.build_blocks(topk, 3, 4, N)
    with pytest.raises(ValueError):
        oracle.build_blocks(np.array([[0, 3]], np.int32), 3, 4, N)


def test_build_blocks_skips_dropped_selections():
    """Page 3's varlen-K routing: a token may activate fewer than K experts; a
    negative id is a dropped selection.  The blocks are those of the routing
    without it (brute force), and a token with every selection dropped owns no
    slot."""
    rng = np.random.default_rng(5)
    T, K, E, B = 60, 3, 5, 8
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    topk[rng.random((T, K)) < 0.3] = -1
    topk[7] = -1
    N = oracle.num_blocks(T, K, E, B)
    tpid, b2e = oracle.build_blocks(topk, E, B, N)
    rt, rb = _reference_blocks(topk, E, B, N)
    assert np.array_equal(tpid, rt) and np.array_equal(b2e, rb)
    assert 7 not in set(tpid.tolist())
    seen = sorted((int(b2e[s // B]), int(tpid[s])) for s in range(N * B) if tpid[s] >= 0)
    assert seen == sorted((int(e), t) for t in range(T) for e in topk[t] if e >= 0)
