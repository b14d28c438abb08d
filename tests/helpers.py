"""Test helpers: assemble oracle problems from the seeded generators.

Only tests import this module.  Quantised weights for the oracle come from the
oracle's own quantiser; nothing here touches the GPU library.
"""
from __future__ import annotations

import numpy as np

import oracle
import synthetic as S


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_F / ||b||_F in float64 (0 when both are 0)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b.ravel())
    na = np.linalg.norm((a - b).ravel())
    if nb == 0.0:
        return 0.0 if na == 0.0 else float("inf")
    return float(na / nb)


def bf(bits) -> np.ndarray:
    return oracle.bf16_to_float(bits).astype(np.float64)


def quantize_weights(w_gate_up_bits: np.ndarray, w_down_bits: np.ndarray, fmt_w: int = oracle.E4M3):
    """Pre-quantise weights along the backward contraction axis:
    W_down [E,I,H] along H, W_gate_up [E,H,2,I] along I (both: the last axis)."""
    E, H, _, I = w_gate_up_bits.shape
    gu_c, gu_s = oracle.quantize(w_gate_up_bits.reshape(E * H * 2, I), 1, fmt_w)
    d_c, d_s = oracle.quantize(w_down_bits.reshape(E * I, H), 1, fmt_w)
    return (gu_c.reshape(E, H, 2, I), gu_s.reshape(E, H, 2, I // 32),
            d_c.reshape(E, I, H), d_s.reshape(E, I, H // 32))


def moe_problem(cfg: S.MoeConfig, nthreads: int = 0, N=None):
    """(oracle.MoeProblem, extras) for a workload config, built on the host."""
    topk, aff = S.routing(cfg)
    if N is None:
        N = oracle.num_blocks(cfg.T, cfg.K, cfg.E, cfg.B)
    tpid, b2e = oracle.build_blocks(topk, cfg.E, cfg.B, N)
    t = S.moe_tensors(cfg, N, "cpu")
    bits = {k: (None if v is None else S.bf16_bits(v)) for k, v in t.items()}
    gu_c, gu_s, d_c, d_s = quantize_weights(bits["w_gate_up"], bits["w_down"])
    p = oracle.MoeProblem(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, N=N, B=cfg.B, hidden=bits["hidden"],
                          aff=aff, wgu_codes=gu_c, wgu_scales=gu_s, wd_codes=d_c, wd_scales=d_s,
                          tpid=tpid, b2e=b2e, dy=bits["dy"], ckpt=bits["ckpt"], b2=bits["b2"],
                          affinity_on=cfg.affinity_on, has_bias=int(cfg.has_bias), nthreads=nthreads)
    return p, dict(topk=topk, bits=bits)


def pairs_to_rows(raw, rows: int, k: int) -> np.ndarray:
    """Scale bytes stored pair-major, [k/128][rows][4] (word (p, r) = row r's
    bytes for elements [128p, 128p+128)), as row-major [rows][k/32]."""
    a = np.asarray(raw, dtype=np.uint8).reshape(k // 128, rows, 4)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(rows, k // 32))


def stage_major_to_rows(raw, rows: int, k: int) -> np.ndarray:
    """Codes of `rows` rows over k elements stored stage-major (the four-slot
    ring's layout: the rows in panels of 256, the last one possibly shorter,
    each panel [k/64][panel rows][64]) as row-major [rows][k]."""
    a = np.asarray(raw, dtype=np.uint8).reshape(-1)
    assert a.size == rows * k and k % 64 == 0
    out = np.empty((rows, k), dtype=np.uint8)
    for p0 in range(0, rows, 256):
        rp = min(256, rows - p0)
        panel = a[p0 * k:(p0 + rp) * k].reshape(k // 64, rp, 64)
        out[p0:p0 + rp] = panel.transpose(1, 0, 2).reshape(rp, k)
    return out


# Localised-defect bounds of the GPU parity checks, next to the relative
# Frobenius bound of the whole tensor (2e-3).  Set from the measured error
# distributions of every parity case with margin; the reasons are in the
# design notes' parity section.
EXPERT_TOL = 4e-3      # relative Frobenius error of one expert's slice (measured worst 6.8e-4)
ROW_TOL = 3e-2         # relative Frobenius error of one output row (measured worst 1.1e-2)
OUTLIER_C = 0.1        # element bound: |g - r| <= OUTLIER_C * rms(r) + 2^-7 |r| (never exceeded)


def parity_stats(g, r, rows=None, experts=None):
    """Error statistics of a GPU tensor g against the oracle's r (float64 arrays).

    rows: the number of rows to view both as (per-row relative error over rows
    whose reference is not all zero); experts: likewise per leading slice.
    Returns dict(rel, row_max, expert_max, outliers) with outliers the count of
    elements past the element bound."""
    g = np.asarray(g, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    out = dict(rel=rel_fro(g, r), row_max=0.0, expert_max=0.0)

    def worst(n):
        if not n or n <= 1:
            return 0.0
        gg, rr = g.reshape(n, -1), r.reshape(n, -1)
        nr = np.linalg.norm(rr, axis=1)
        ne = np.linalg.norm(gg - rr, axis=1)
        live = nr > 0
        return float((ne[live] / nr[live]).max()) if live.any() else 0.0

    out["row_max"] = worst(rows)
    out["expert_max"] = worst(experts)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    out["outliers"] = int(np.count_nonzero(np.abs(g - r) > OUTLIER_C * rms + 2.0 ** -7 * np.abs(r)))
    return out


def assert_parity(name, st, tol=2e-3, row_tol=ROW_TOL, expert_tol=EXPERT_TOL):
    assert st["rel"] <= tol, (name, "relative Frobenius", st)
    assert st["row_max"] <= row_tol, (name, "worst row", st)
    assert st["expert_max"] <= expert_tol, (name, "worst expert", st)
    assert st["outliers"] == 0, (name, "elements past the element bound", st)


def rows_to_pairs(scales, rows: int, k: int) -> np.ndarray:
    """Row-major scale bytes [rows][k/32] packed pair-major, [k/128][rows][4]
    (the inverse of pairs_to_rows)."""
    a = np.asarray(scales, dtype=np.uint8).reshape(rows, k // 128, 4)
    return np.ascontiguousarray(a.transpose(1, 0, 2))
