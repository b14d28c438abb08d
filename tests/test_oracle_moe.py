"""Pins of the oracle's MoE backward.

Exact mode (fp64, no quantisation) against central finite differences of its own
forward and against torch autograd of an independently written forward.  MXFP8
mode against: the exact mode (with quantisation switched off, and within the
quantisation noise with it on), the dense backward through the single-expert
identity (bit-exact), power-of-two equivariance in dY, padding invariance, empty
experts, and its own restricted evaluators.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import bf, moe_problem, quantize_weights, rel_fro


def _bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _routing(rng, T, K, E, B, N=None):
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    tpid, b2e = oracle.build_blocks(topk, E, B, N)
    aff = np.zeros((T, E))
    for t in range(T):
        aff[t, topk[t]] = rng.uniform(0.1, 1.0, K)
    return topk, tpid, b2e, aff.reshape(-1)


def _exact_problem(rng, T=10, H=6, I=5, E=3, K=2, B=4, bias=True, on=0, act=0):
    topk, tpid, b2e, aff = _routing(rng, T, K, E, B)
    return oracle.MoeExact(
        x=rng.standard_normal((T, H)), aff=aff, wgu=rng.standard_normal((E, H, 2, I)) * 0.5,
        wd=rng.standard_normal((E, I, H)) * 0.5, tpid=tpid, b2e=b2e, B=B,
        b1=rng.standard_normal((E, 2, I)) * 0.3 if bias else None,
        b2=rng.standard_normal((E, H)) * 0.3 if (bias and on == 0) else None, affinity_on=on, activation=act)


@pytest.mark.parametrize("on,act", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_exact_mode_finite_differences(on, act):
    rng = np.random.default_rng(20 + on + 10 * act)
    p = _exact_problem(rng, on=on, act=act)
    T, H = p.x.shape
    dy = rng.standard_normal((T, H))
    g = oracle.moe_bwd_exact(p, dy)
    names = [("x", "dx"), ("aff", "daff"), ("wgu", "dwgu"), ("wd", "dwd"), ("b1", "db1")]
    if on == 0:
        names.append(("b2", "db2"))
    h = 1e-6
    for pname, gname in names:
        base = getattr(p, pname)
        fd = np.zeros(base.size)
        for j in range(base.size):
            for sgn in (1, -1):
                pert = base.copy().reshape(-1)
                pert[j] += sgn * h
                setattr(p, pname, pert.reshape(base.shape))
                fd[j] += sgn * np.sum(dy * oracle.moe_fwd_exact(p))
            fd[j] /= 2 * h
        setattr(p, pname, base)
        ana = g[gname].reshape(-1)
        err = np.max(np.abs(fd - ana)) / max(1.0, np.max(np.abs(ana)))
        assert err < 1e-7, (pname, err)


@pytest.mark.parametrize("act", [0, 1])
def test_exact_mode_matches_torch_autograd(act):
    """A forward written directly in torch (per token, over its chosen experts),
    differentiated by autograd in float64 on the CPU.  GeGLU uses torch's GELU
    in its erf form (approximate='none'); the tanh form differs by ~1e-3, far
    past this test's tolerance, so the reading of GELU is pinned here."""
    rng = np.random.default_rng(23)
    p = _exact_problem(rng, T=12, H=7, I=6, E=4, K=2, B=4, act=act)
    gate = torch.nn.functional.silu if act == 0 else (lambda v: torch.nn.functional.gelu(v, approximate="none"))
    T, H = p.x.shape
    E = p.wgu.shape[0]
    dy = rng.standard_normal((T, H))
    tp = {k: torch.tensor(getattr(p, k), dtype=torch.float64, requires_grad=True)
          for k in ("x", "aff", "wgu", "wd", "b1", "b2")}
    routed = [(int(p.tpid[s]), int(p.b2e[s // p.B])) for s in range(p.tpid.size) if p.tpid[s] >= 0]
    y = torch.zeros(T, H, dtype=torch.float64)
    for t, e in routed:
        gu = tp["x"][t] @ tp["wgu"][e].reshape(H, -1)
        gu = gu.reshape(2, -1) + tp["b1"][e]
        inter = gate(gu[0]) * gu[1]
        y = y.index_add(0, torch.tensor([t]), (tp["aff"][t * E + e] * (inter @ tp["wd"][e] + tp["b2"][e]))[None])
    (y * torch.from_numpy(dy)).sum().backward()
    g = oracle.moe_bwd_exact(p, dy)
    for k, gk in (("x", "dx"), ("aff", "daff"), ("wgu", "dwgu"), ("wd", "dwd"), ("b1", "db1"), ("b2", "db2")):
        np.testing.assert_allclose(g[gk], tp[k].grad.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- MX mode
def _mx_and_exact(rng, T=24, H=64, I=64, E=3, K=2, B=32, on=0, bias=True, fmt_act=0, fmt_grad=1, act=0):
    """An MX problem and the exact problem it approximates: same routing, bf16
    activations, dequantised weights, checkpoint = bf16 of the exact pre-activations."""
    topk, tpid, b2e, aff = _routing(rng, T, K, E, B)
    aff = aff.astype(np.float32)
    x = _bits(rng.standard_normal((T, H)))
    dy = _bits(rng.standard_normal((T, H)))
    wgu = _bits(rng.standard_normal((E, H, 2, I)) * 0.1)
    wd = _bits(rng.standard_normal((E, I, H)) * 0.1)
    b1 = rng.standard_normal((E, 2, I)) * 0.1
    b2 = _bits(rng.standard_normal((E, H)) * 0.1) if (bias and on == 0) else None
    gu_c, gu_s, d_c, d_s = quantize_weights(wgu, wd)
    ex = oracle.MoeExact(x=bf(x), aff=aff.astype(np.float64),
                         wgu=oracle.dequantize(gu_c.reshape(-1, I), gu_s.reshape(-1, I // 32), 1, 0).reshape(E, H, 2, I),
                         wd=oracle.dequantize(d_c.reshape(-1, H), d_s.reshape(-1, H // 32), 1, 0).reshape(E, I, H),
                         tpid=tpid, b2e=b2e, B=B, b1=b1, b2=None if b2 is None else bf(b2), affinity_on=on,
                         activation=act)
    _, ck = oracle.moe_fwd_exact(ex, want_ckpt=True)
    mx = oracle.MoeProblem(T=T, H=H, I=I, E=E, N=b2e.size, B=B, hidden=x, aff=aff, wgu_codes=gu_c,
                           wgu_scales=gu_s, wd_codes=d_c, wd_scales=d_s, tpid=tpid, b2e=b2e, dy=dy,
                           ckpt=_bits(ck), b2=b2, affinity_on=on, has_bias=int(b2 is not None),
                           fmt_act=fmt_act, fmt_grad=fmt_grad, activation=act)
    return mx, ex, bf(dy)


KEYS = ("dx", "daff", "dwgu", "dwd", "db1", "db2")


@pytest.mark.parametrize("on,act", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_mx_mode_without_quantisation_matches_exact(on, act):
    """Activation and gradient quantisation switched off: only bf16 rounding points
    remain, so the quantised path's algebra must reproduce the exact gradients."""
    rng = np.random.default_rng(30 + on)
    mx, ex, dy = _mx_and_exact(rng, on=on, fmt_act=oracle.NONE, fmt_grad=oracle.NONE, act=act)
    got = oracle.moe_bwd(mx)
    ref = oracle.moe_bwd_exact(ex, dy)
    for k in KEYS:
        if on == 1 and k == "db2":
            continue
        assert rel_fro(bf(got[k]).reshape(ref[k].shape), ref[k]) < 1e-2, k


@pytest.mark.parametrize("on,act", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_mx_mode_within_quantisation_noise(on, act):
    rng = np.random.default_rng(32 + on)
    mx, ex, dy = _mx_and_exact(rng, on=on, act=act)
    got = oracle.moe_bwd(mx)
    ref = oracle.moe_bwd_exact(ex, dy)
    for k in ("dx", "daff", "dwgu", "dwd", "db1"):
        e = rel_fro(bf(got[k]).reshape(ref[k].shape), ref[k])
        assert 1e-3 < e < 0.15, (k, e)        # e5m2/e4m3 noise is a few percent


@pytest.mark.parametrize("on", [0, 1])
def test_single_expert_identity_with_dense(on):
    """E=1, K=1, affinity 1, tokens in order: each phase equals the dense MXFP8
    backward of the matching operands, bit for bit."""
    rng = np.random.default_rng(40 + on)
    T, H, I, B = 64, 64, 96, 32
    topk = np.zeros((T, 1), np.int32)
    tpid, b2e = oracle.build_blocks(topk, 1, B)
    assert np.array_equal(tpid, np.arange(T))
    x = _bits(rng.standard_normal((T, H)))
    dy = _bits(rng.standard_normal((T, H)))
    wgu = _bits(rng.standard_normal((1, H, 2, I)) * 0.1)
    wd = _bits(rng.standard_normal((1, I, H)) * 0.1)
    ck = _bits(rng.standard_normal((b2e.size, 2, I, B)))
    gu_c, gu_s, d_c, d_s = quantize_weights(wgu, wd)
    mx = oracle.MoeProblem(T=T, H=H, I=I, E=1, N=b2e.size, B=B, hidden=x, aff=np.ones(T, np.float32),
                           wgu_codes=gu_c, wgu_scales=gu_s, wd_codes=d_c, wd_scales=d_s, tpid=tpid,
                           b2e=b2e, dy=dy, ckpt=ck, affinity_on=on)
    out = oracle.moe_bwd(mx)
    det = [oracle.moe_block_detail(mx, b) for b in range(b2e.size)]
    dS = np.concatenate([d["dS"] for d in det])
    dgu = np.concatenate([np.concatenate([d["dG"], d["dU"]], 1) for d in det])     # [T, 2I]
    inter = np.concatenate([d["inter"] for d in det])
    wd_deq = oracle.dequantize(d_c.reshape(I, H), d_s.reshape(I, H // 32), 1, 0)    # [I, H]
    wgu_deq = oracle.dequantize(gu_c.reshape(H * 2, I), gu_s.reshape(H * 2, I // 32), 1, 0).reshape(H, 2 * I)
    wd_b, wgu_b = _bits(wd_deq), _bits(wgu_deq)
    assert np.array_equal(bf(wd_b), wd_deq) and np.array_equal(bf(wgu_b), wgu_deq)   # weights exact in bf16
    # Phase 1: dS = Q_H(dY) . Q_H(W_down)^T  ==  dense dX with W = W_down^T
    d1, _ = oracle.dense_bwd(dy, np.ascontiguousarray(wd_b.T), x, want_dw=False)
    assert np.array_equal(d1, _bits(dS))
    # Phase 3: dX = Q_I(dGU) . Q_I(W_gu)^T  ==  dense dX with W = W_gu viewed [2I, H]
    d3, _ = oracle.dense_bwd(dgu, np.ascontiguousarray(wgu_b.T), x, want_dw=False)
    assert np.array_equal(d3, out["dx"])
    # Phase 2: dW_gu = Q_tok(X)^T . Q_tok(dGU)  ==  dense dW [2I, H]
    _, d2 = oracle.dense_bwd(dgu, np.zeros((2 * I, H), np.uint16), x, want_dx=False)
    assert np.array_equal(d2, out["dwgu"][0].reshape(H, 2 * I).T)
    # Phase 4 (a = 1 so a*dY = dY and a*inter = inter): dense dW with dY' = inter, X' = dY
    _, d4 = oracle.dense_bwd(inter, np.zeros((I, H), np.uint16), dy, fmt_dy=oracle.E4M3,
                             fmt_x=oracle.E5M2, want_dx=False)
    assert np.array_equal(d4, out["dwd"][0])


def test_dy_power_of_two_equivariance():
    rng = np.random.default_rng(50)
    mx, _, _ = _mx_and_exact(rng, on=0, bias=True)
    base = oracle.moe_bwd(mx)
    mx.dy = _bits(bf(mx.dy) * 8.0)
    scaled = oracle.moe_bwd(mx)
    for k in KEYS:
        assert np.array_equal(bf(scaled[k]), 8.0 * bf(base[k])), k


def test_padding_blocks_and_pad_checkpoint_ignored():
    cfg = S.scaled(S.TINY, T=96, I=64, H=64)
    p, _ = moe_problem(cfg)
    base = oracle.moe_bwd(p)
    N2 = p.N + 2
    p2, _ = moe_problem(cfg, N=N2)
    rng = np.random.default_rng(51)
    ck = p2.ckpt.copy()
    pad = p2.tpid.reshape(N2, 1, 1, cfg.B) < 0
    ck[np.broadcast_to(pad, ck.shape)] = rng.integers(0, 1 << 16, np.count_nonzero(np.broadcast_to(pad, ck.shape)),
                                                      dtype=np.uint16) & 0x7F7F
    p2.ckpt = ck
    other = oracle.moe_bwd(p2)
    for k in KEYS:
        assert np.array_equal(base[k], other[k]), k


def test_empty_expert_and_restricted_evaluators():
    cfg = S.scaled(S.FINE, T=64, H=64, I=64, E=12, K=2, B=32)
    p, ex = moe_problem(cfg)
    cnt = np.bincount(ex["topk"].ravel(), minlength=cfg.E)
    assert (cnt == 0).any()
    full = oracle.moe_bwd(p)
    for e in np.nonzero(cnt == 0)[0]:
        for k in ("dwgu", "dwd", "db1", "db2"):
            assert not bf(full[k][e]).any(), (k, e)
    tok = np.array([3, 0, 63, 17])
    dx, da = oracle.moe_token_rows(p, tok)
    assert np.array_equal(dx, full["dx"][tok])
    assert np.array_equal(da, full["daff"].reshape(cfg.T, cfg.E)[tok])
    e = int(np.argmax(cnt))
    cols = np.array([5, 0, 63, 31])
    r = oracle.moe_expert_cols(p, e, cols)
    assert np.array_equal(r["dwgu"], full["dwgu"][e][:, :, cols])
    assert np.array_equal(r["dwd"], full["dwd"][e][cols])
    assert np.array_equal(r["db1"], full["db1"][e][:, cols])
    assert np.array_equal(r["db2"], full["db2"][e])
    # unrouted (token, expert) pairs get a zero affinity gradient
    routed = np.zeros((cfg.T, cfg.E), bool)
    routed[np.arange(cfg.T)[:, None], ex["topk"]] = True
    assert not bf(full["daff"].reshape(cfg.T, cfg.E)[~routed]).any()


def test_affinity_placement_changes_only_dw_down():
    rng = np.random.default_rng(52)
    mx, _, _ = _mx_and_exact(rng, on=0, bias=False)
    a = oracle.moe_bwd(mx)
    mx.affinity_on = 1
    b = oracle.moe_bwd(mx)
    for k in ("dx", "daff", "dwgu", "db1", "db2"):
        assert np.array_equal(a[k], b[k]), k
    assert not np.array_equal(a["dwd"], b["dwd"])
    assert rel_fro(bf(a["dwd"]), bf(b["dwd"])) < 0.1


def test_token_operands_match_their_definition():
    """The token-axis operands read back from the oracle are the 32-slot groups of
    the gathered values (X rows, and a*dY under affinity on H)."""
    cfg = S.scaled(S.TINY, T=64, I=64, H=64)
    p, _ = moe_problem(cfg)
    P = p.N * p.B
    codes, scales = oracle.moe_token_operand(p, oracle.TOK_X)
    gathered = np.zeros((P, p.H), np.uint16)
    valid = (p.tpid >= 0) & (p.tpid < p.T)
    gathered[valid] = p.hidden[p.tpid[valid]]
    c2, s2 = oracle.quantize(np.ascontiguousarray(gathered.T), 1, oracle.E4M3)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    codes, scales = oracle.moe_token_operand(p, oracle.TOK_GY)
    e = p.b2e[np.arange(P) // p.B]
    a = np.where(valid, p.aff[np.where(valid, p.tpid, 0) * p.E + e], 0).astype(np.float32)
    gy = np.zeros((P, p.H), np.float32)
    gy[valid] = a[valid, None] * bf(p.dy[p.tpid[valid]]).astype(np.float32)      # fp32 product
    c2, s2 = oracle.quantize(np.ascontiguousarray(_bits(gy).T), 1, oracle.E5M2)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)


def test_accumulate_adds_into_the_outputs():
    """P1's accumulation flag (reading: add into the gradients).  Pins: with zero
    priors it is the overwrite result bit for bit; onto the negated overwrite
    result only the rounding residual g - bf16(g) is left (|.| <= 2^-8 |g|),
    which fails if the prior were ignored, replaced or subtracted, output by
    output; the restricted evaluators accumulate the same way."""
    cfg = S.scaled(S.FINE, T=64, H=64, I=64, E=6, K=2, B=32)
    p, ex = moe_problem(cfg)
    assert p.has_bias
    base = oracle.moe_bwd(p)
    p.accumulate = 1
    zero = oracle.moe_bwd(p, prior={k: np.zeros_like(v) for k, v in base.items()})
    for k in KEYS:
        assert np.array_equal(base[k], zero[k]), k
    neg = {k: v ^ np.uint16(0x8000) for k, v in base.items()}
    res = oracle.moe_bwd(p, prior=neg)
    for k in KEYS:
        g, r = bf(base[k]), bf(res[k])
        assert np.all(np.abs(r) <= 2.0 ** -8 * np.abs(g)), k
        assert np.abs(g).max() > 0, k
    # a prior of other values: within one rounding of prior + bf16(g)
    rng = np.random.default_rng(53)
    prior = {k: oracle_bits(rng.standard_normal(v.shape) * np.abs(bf(v)).max()) for k, v in base.items()}
    acc = oracle.moe_bwd(p, prior=prior)
    for k in KEYS:
        want = bf(prior[k]) + bf(base[k])
        tol = 2.0 ** -8 * (np.abs(want) + np.abs(bf(base[k]))) + 1e-30
        assert np.all(np.abs(bf(acc[k]) - want) <= tol), k
    tok = np.array([5, 0, 63])
    dx, da = oracle.moe_token_rows(p, tok, prior=dict(dx=prior["dx"][tok],
                                                      daff=prior["daff"].reshape(cfg.T, cfg.E)[tok]))
    assert np.array_equal(dx, acc["dx"][tok])
    assert np.array_equal(da, acc["daff"].reshape(cfg.T, cfg.E)[tok])
    e, cols = 1, np.array([3, 63, 0])
    r = oracle.moe_expert_cols(p, e, cols, prior=dict(dwgu=prior["dwgu"][e][:, :, cols], dwd=prior["dwd"][e][cols],
                                                      db1=prior["db1"][e][:, cols], db2=prior["db2"][e]))
    assert np.array_equal(r["dwgu"], acc["dwgu"][e][:, :, cols])
    assert np.array_equal(r["dwd"], acc["dwd"][e][cols])
    assert np.array_equal(r["db1"], acc["db1"][e][:, cols])
    assert np.array_equal(r["db2"], acc["db2"][e])


def oracle_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (one RNE rounding)."""
    return np.vectorize(oracle.double_to_bf16, otypes=[np.uint16])(x)


@pytest.mark.parametrize("on", [0, 1])
def test_token_operands_of_the_epilogue_match_their_definition(on):
    """The other two token-axis operands: the intermediate (mode 2; under the
    affinity on I it is bf16(fp32(a * intermediate))) and [dGate; dUp] (mode 3),
    each the 32-slot groups of the per-slot values gathered into [rows, P].
    The per-slot values come from the block evaluator, whose arithmetic the
    single-expert identity and the finite-difference pins fix; this pins the
    gather, the row order (gate rows before up rows), the affinity product and
    its rounding, the format and the group axis."""
    cfg = S.scaled(S.TINY, T=64, I=64, H=64, E=4, K=2, B=32)
    p, _ = moe_problem(cfg)
    p.affinity_on = on
    P = p.N * p.B
    valid = (p.tpid >= 0) & (p.tpid < p.T)
    e = p.b2e[np.arange(P) // p.B]
    a = np.where(valid, p.aff[np.where(valid, p.tpid, 0) * p.E + e], 0).astype(np.float32)
    det = [oracle.moe_block_detail(p, b) for b in range(p.N)]
    inter = np.concatenate([d["inter"] for d in det])                       # [P, I] bf16 bits
    dgu = np.concatenate([np.concatenate([d["dG"], d["dU"]], 1) for d in det])   # [P, 2I]
    inter[~valid] = 0
    dgu[~valid] = 0
    if on == 1:
        inter = _bits(a[:, None] * bf(inter).astype(np.float32))           # fp32 product, one bf16 rounding
    codes, scales = oracle.moe_token_operand(p, oracle.TOK_INTER)
    c2, s2 = oracle.quantize(np.ascontiguousarray(inter.T), 1, oracle.E4M3)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    codes, scales = oracle.moe_token_operand(p, oracle.TOK_DGU)
    c2, s2 = oracle.quantize(np.ascontiguousarray(dgu.T), 1, oracle.E5M2)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # the affinity really enters mode 2 under the affinity on I (and only there)
    assert (on == 1) != np.array_equal(
        oracle.moe_token_operand(p, oracle.TOK_INTER)[0],
        oracle.quantize(np.ascontiguousarray(np.concatenate([d["inter"] for d in det]).T * valid[None]
                                             .astype(np.uint16)), 1, oracle.E4M3)[0])


def test_geglu_changes_only_what_the_gate_activation_reaches():
    """Same problem under SwiGLU and GeGLU: every gradient that passes through
    the gate activation changes, and the per-slot activation values are the
    bf16 roundings of silu(g) and of g * Phi(g) (erf form) of the checkpoint."""
    import math
    rng = np.random.default_rng(54)
    mx, _, _ = _mx_and_exact(rng, on=0, bias=True)
    a = oracle.moe_bwd(mx)
    mx.activation = oracle.GEGLU
    b = oracle.moe_bwd(mx)
    for k in ("dx", "daff", "dwgu", "dwd", "db1"):
        assert not np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["db2"], b["db2"])           # a * dY does not see the activation
    d = oracle.moe_block_detail(mx, 0)
    g = bf(mx.ckpt[0, 0].T)                             # [B, I] gate pre-activations of block 0
    valid = mx.tpid[:mx.B] >= 0
    want = np.vectorize(lambda v: oracle.double_to_bf16(0.5 * v * math.erfc(-v / math.sqrt(2.0))),
                        otypes=[np.uint16])(g)
    assert np.array_equal(d["ga"][valid], want[valid])
