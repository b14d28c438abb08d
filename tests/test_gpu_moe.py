"""moe_bwd_mxfp8 (and moe_build_blocks) on the GPU against the oracle.

Bar: routing blocks, weight codes and the quantised input operands (dY rows,
gathered X and a*dY along slots) bit-exact; every gradient within relative
Frobenius error 2e-3; exact zeros where the oracle is zero (unrouted pairs,
empty experts)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import assert_parity, bf, pairs_to_rows, parity_stats, rel_fro, stage_major_to_rows
from moe_gpu_common import gpu_problem, host, oracle_problem

pytestmark = pytest.mark.gpu
TOL = 2e-3

SMALL = {
    "tiny": S.TINY,
    "medium_s": S.scaled(S.MEDIUM, T=512, H=256, I=352, E=8, K=4, B=128),
    "large_s": S.scaled(S.LARGE, T=256, H=256, I=512, E=4, K=2, B=256),
    "fine_s": S.scaled(S.FINE, T=512, H=192, I=128, E=16, K=4, B=128),
    "medium_b512": S.scaled(S.MEDIUM, T=640, H=128, I=96, E=4, K=2, B=512),
    # H a multiple of 128: the bias reductions ride on the dY gather
    "fine_h256": S.scaled(S.FINE, T=512, H=256, I=128, E=16, K=4, B=128),
    # stage-major operands whose rows end in a short 256-row panel: X and dY over
    # H = 384 (256 + 128), dGU over 2I = 384, the intermediate over I = 192
    "ragged_panels": S.scaled(S.MEDIUM, T=384, H=384, I=192, E=4, K=2, B=128),
    # 2I = 4096 with 2 MiB experts: Phase 3 cuts its tiles (all in one partial
    # round) along K in the contiguous tile order
    "cut_contiguous": S.scaled(S.MEDIUM, T=512, H=256, I=2048, E=4, K=2, B=256),
}
# experts of 32 MiB (W_down) and 64 MiB (W_gate_up): Phases 1 and 3 hand their
# tiles to the XCDs round robin, which no other small case reaches; with 2I =
# 16384 and fewer tiles than CUs, Phase 3 also cuts every tile along K into
# parts summed afterwards
ROUND_ROBIN = {"large_rr": S.scaled(S.LARGE, T=256, H=4096, I=8192, E=2, K=1, B=128)}


def _views(cfg):
    """(rows, experts) to view each gradient as: per-token rows of dX and d(a);
    per-expert slices and their rows of the weight and bias gradients."""
    E, H, I, T = cfg.E, cfg.H, cfg.I, cfg.T
    return {"dx": (T, None), "daff": (T, None), "dwgu": (E * H, E), "dwd": (E * I, E), "db1": (E * 2, E),
            "db2": (E, E)}


def _check_outputs(cfg, out, ref, unrouted_zero=True, zero_keys=None):
    """Whole-tensor relative Frobenius error <= 2e-3 for every gradient, plus the
    localised bounds of helpers.assert_parity (worst expert slice, worst row,
    element outliers) and exact zeros where the oracle is exactly zero."""
    keys = ["dx", "daff", "dwgu", "dwd"] + (["db1", "db2"] if cfg.has_bias else [])
    stats = {}
    views = _views(cfg)
    for k in keys:
        g = bf(host(out[k])).reshape(-1)
        r = bf(ref[k]).reshape(-1)
        rows, experts = views[k]
        stats[k] = parity_stats(g, r, rows=rows, experts=experts)
        if unrouted_zero and (zero_keys is None or k in zero_keys):
            assert np.all(g[r == 0] == 0) or k in ("dx",), f"{k}: nonzero where the oracle is exactly zero"
    print(cfg.name, {k: {a: (f"{b:.2e}" if isinstance(b, float) else b) for a, b in v.items()}
                     for k, v in stats.items()}, flush=True)
    for k, st in stats.items():
        assert_parity(k, st, tol=TOL)


@pytest.mark.parametrize("name", list(SMALL) + list(ROUND_ROBIN))
def test_moe_small_full_parity(name):
    cfg = {**SMALL, **ROUND_ROBIN}[name]
    gp = gpu_problem(cfg)
    out = gp["op"].run()
    torch.cuda.synchronize()
    p, ex = oracle_problem(gp)
    # routing blocks and weight codes: bit-exact
    assert np.array_equal(host(gp["tpid"]), ex["tpid"]) and np.array_equal(host(gp["b2e"]), ex["b2e"])
    for g, o in zip(gp["wq"], ex["wq"]):
        assert np.array_equal(host(g).reshape(-1), o.reshape(-1))
    ref = oracle.moe_bwd(p)
    # large_rr and cut_contiguous have no empty expert, so their only structural
    # zeros are the unrouted d(a) pairs; with 128-256 slots per expert and long
    # I the oracle's exact dW sums can also cancel to 0 by chance (23 of 134M
    # dW_gate_up entries in large_rr), where a rare one-step difference in a
    # dGate/dUp code leaves a residue
    daff_zeros_only = name in ROUND_ROBIN or name == "cut_contiguous"
    _check_outputs(cfg, out, ref, zero_keys=("daff",) if daff_zeros_only else None)
    # quantised input operands read back from the workspace: bit-exact
    op = gp["op"]
    T, H, P = cfg.T, cfg.H, gp["N"] * cfg.B
    ws = op.workspace.cpu().numpy()
    L = op.layout
    c, s = oracle.quantize(p.dy, 1, oracle.E5M2)
    assert np.array_equal(ws[L["dy_codes"]:L["dy_codes"] + T * H], c.ravel())
    got = ws[L["dy_scales"]:L["dy_scales"] + T * H // 32]
    if H % 128 == 0:   # pair-major ([H/128][T][4]) when Phase 1 streams the codes
        got = pairs_to_rows(got, T, H)
    assert np.array_equal(got.ravel(), s.ravel())
    for which, name_c, name_s in ((oracle.TOK_X, "x_tok_codes", "x_tok_scales"),
                                  (oracle.TOK_GY, "gy_tok_codes", "gy_tok_scales")):
        c, s = oracle.moe_token_operand(p, which)
        # token-axis codes are stage-major (H rows over P slots)
        assert np.array_equal(stage_major_to_rows(ws[L[name_c]:L[name_c] + H * P], H, P), c.reshape(H, P)), name_c
        # token-axis scales are pair-major ([P/128][H][4])
        got = pairs_to_rows(ws[L[name_s]:L[name_s] + H * P // 32], H, P)
        assert np.array_equal(got, s.reshape(H, P // 32)), name_s
    # the weights' scales re-laid pair-major for the ring loops: the oracle's bytes
    _, gu_s, _, d_s = ex["wq"]
    E, I = cfg.E, cfg.I
    if (2 * I) % 128 == 0:
        raw = ws[L["wgu_scales_pairs"]:L["wgu_scales_pairs"] + E * H * 2 * I // 32].reshape(E, -1)
        for e in range(E):
            assert np.array_equal(pairs_to_rows(raw[e], H, 2 * I), gu_s.reshape(E, H, 2 * I // 32)[e]), e
    if H % 128 == 0:
        raw = ws[L["wd_scales_pairs"]:L["wd_scales_pairs"] + E * I * H // 32].reshape(E, -1)
        for e in range(E):
            assert np.array_equal(pairs_to_rows(raw[e], I, H), d_s.reshape(E, I, H // 32)[e]), e
    # the intermediate operand: silu is evaluated in fp32 on the GPU and in fp64 by the
    # oracle, so a rare bf16 rounding may differ; codes must agree almost everywhere
    c, s = oracle.moe_token_operand(p, oracle.TOK_INTER)
    got = stage_major_to_rows(ws[L["inter_tok_codes"]:L["inter_tok_codes"] + cfg.I * P], cfg.I, P)
    assert np.mean(got != c.reshape(cfg.I, P)) < 1e-3
    # dGate|dUp along the slots (Phase 2's operand), with the same caveat, at the
    # routed slots (blocks without any are never written: no GEMM reads them)
    c, s = oracle.moe_token_operand(p, oracle.TOK_DGU)
    got = stage_major_to_rows(ws[L["dgu_tok_codes"]:L["dgu_tok_codes"] + 2 * cfg.I * P], 2 * cfg.I, P)
    tp = host(gp["tpid"]).reshape(-1)
    routed = (tp >= 0) & (tp < T)
    assert routed.any()
    assert np.mean(got[:, routed] != c.reshape(2 * cfg.I, P)[:, routed]) < 1e-3


def test_moe_build_blocks_bit_exact_and_edge_cases():
    import mxfp8_grouped_gemm_amd as mx
    rng = np.random.default_rng(3)
    # (70000, 4, 1024, ...) places 9 rounds of 256 tokens per chunk with the most experts the
    # per-chunk LDS kernels take; (20000, 8, 2048, ...) takes the per-(expert, chunk) kernels
    for T, K, E, B in ((1000, 3, 7, 128), (64, 1, 64, 128), (4096, 8, 128, 128), (300, 2, 3, 1024),
                       (70000, 4, 1024, 128), (20000, 8, 2048, 128)):
        topk = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        if E == 7:
            topk[topk == 5] = 4 if K == 1 else topk[topk == 5]      # keep rows distinct
        N = oracle.num_blocks(T, K, E, B) + 2                        # extra trailing blocks
        tp, be = mx.moe_build_blocks(torch.from_numpy(topk).cuda(), E, B, N)
        rt, rb = oracle.build_blocks(topk, E, B, N)
        assert np.array_equal(host(tp), rt) and np.array_equal(host(be), rb)
    with pytest.raises(mx.MxError):
        mx.moe_build_blocks(torch.zeros((4, 2), dtype=torch.int32, device="cuda"), 4, 128, 1)


@pytest.mark.parametrize("name", ["fine_s", "cut_contiguous"])
def test_moe_deterministic_weight_grads_and_dy_scaling(name):
    """Phases 2/4, the per-token dX sums, Phase 3's cut tiles (cut_contiguous)
    and the d(a) partials have a fixed summation order: repeated runs give
    identical dW, dX and d(a), and scaling dY by 2^3 scales them by exactly 8
    (the E8M0 scales absorb it).  The bias sums use atomics."""
    cfg = SMALL[name]
    gp = gpu_problem(cfg)
    a = {k: v.clone() for k, v in gp["op"].run().items() if v is not None}
    b = gp["op"].run()
    for k in ("dwgu", "dwd", "dx", "daff"):
        assert torch.equal(a[k], b[k]), k
    bias = ("db1", "db2") if cfg.has_bias else ()
    for k in bias:
        assert rel_fro(bf(host(b[k])), bf(host(a[k]))) < 1e-5, k
    gp["t"]["dy"].mul_(8.0)
    c = gp["op"].run()
    for k in ("dwgu", "dwd", "dx", "daff"):
        assert torch.equal(c[k].float(), 8.0 * a[k].float()), k
    for k in bias:
        assert rel_fro(bf(host(c[k])), 8.0 * bf(host(a[k]))) < 1e-5, k


def test_moe_extra_padding_blocks_change_nothing():
    cfg = SMALL["tiny"]
    g1 = gpu_problem(cfg)
    o1 = {k: v.clone() for k, v in g1["op"].run().items() if v is not None}
    g2 = gpu_problem(cfg, N=g1["N"] + 3)
    o2 = g2["op"].run()
    for k in ("dwgu", "dwd", "dx", "daff"):
        assert torch.equal(o1[k], o2[k]), k


def test_moe_rejects_bad_arguments():
    import mxfp8_grouped_gemm_amd as mx
    gp = gpu_problem(SMALL["tiny"])
    args = gp["op"].args
    saved = args.block_size
    args.block_size = 96
    with pytest.raises(mx.MxError) as ei:
        gp["op"].run()
    assert ei.value.status == 2
    args.block_size = saved
    args.affinity_on = 1
    args.has_bias = 1
    with pytest.raises(mx.MxError):
        gp["op"].run()
    args.affinity_on, args.has_bias = 0, 0
    # a workspace below the size query: MXFP8_ERR_WORKSPACE, nothing enqueued
    assert mx.lib().moe_bwd_mxfp8(mx.C.byref(args), gp["op"].workspace.data_ptr(), 1024, None) == 3
    assert "workspace" in mx.last_error()
    gp["op"].run()      # still works after the failed calls


# ----------------------------------------------------------------------------- full sizes, sampled
FULL = {"medium": S.MEDIUM, "large": S.LARGE, "fine": S.FINE}


@pytest.mark.parametrize("name", list(FULL))
def test_moe_full_size_sampled(name):
    """The benchmark's sizes and launch configuration.  The oracle computes
    sampled outputs: whole dX rows and d(a) entries of 26 tokens, and whole dW
    columns / rows of 8 intermediate indices of three experts."""
    _check_sampled(FULL[name], name)


def test_moe_bf16_inputs_over_2gib_sampled():
    """X and dY of 2.1 GB each (T * H * 2 above 2^31): the gathers along the
    slots read them at 64-bit addresses and the bias reductions run in their
    own kernels.  Sampled as at the full sizes."""
    cfg = S.scaled(S.FINE, T=262400, H=4096, I=256, E=8, K=1, B=512)
    assert cfg.T * cfg.H * 2 > 2**31 - 1 and cfg.has_bias
    _check_sampled(cfg, "over_2gib")


def _check_sampled(cfg, name):
    print(f"{name}: {cfg.name}", flush=True)
    gp = gpu_problem(cfg)
    out = gp["op"].run()
    torch.cuda.synchronize()
    print(f"{name}: GPU run done", flush=True)
    p, ex = oracle_problem(gp)
    assert np.array_equal(host(gp["tpid"]), ex["tpid"]) and np.array_equal(host(gp["b2e"]), ex["b2e"])
    rng = np.random.default_rng(1)
    cnt = np.bincount(gp["topk"].ravel(), minlength=cfg.E)
    # plus the tokens of the last two routed slots: the last live block's last
    # slot tile, in Phase 3's last round of tiles (cut along K at long 2I)
    tp = host(gp["tpid"]).reshape(-1)
    routed = np.nonzero((tp >= 0) & (tp < cfg.T))[0]
    tokens = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 22),
                                       tp[routed[-2:]]])).astype(np.int32)
    dx_r, da_r = oracle.moe_token_rows(p, tokens)
    gdx = bf(host(out["dx"]))[tokens]
    gda = bf(host(out["daff"])).reshape(cfg.T, cfg.E)[tokens]
    e_dx, e_da = rel_fro(gdx, bf(dx_r)), rel_fro(gda, bf(da_r))
    assert np.all(gda[bf(da_r) == 0] == 0)
    local = {"dx": parity_stats(gdx, bf(dx_r), rows=len(tokens)),
             "daff": parity_stats(gda, bf(da_r), rows=len(tokens))}
    # the busiest, the least busy and a median expert (among those with tokens)
    live = np.nonzero(cnt > 0)[0]
    experts = sorted({int(np.argmax(cnt)), int(live[np.argmin(cnt[live])]),
                      int(live[np.argsort(cnt[live])[len(live) // 2]])})
    icols = np.unique(np.concatenate([[0, cfg.I - 1], rng.integers(0, cfg.I, 6)])).astype(np.int32)
    errs = {"dx": e_dx, "daff": e_da}
    for e in experts:
        r = oracle.moe_expert_cols(p, e, icols)
        errs[f"dwgu[{e}]"] = rel_fro(bf(host(out["dwgu"][e]))[:, :, icols], bf(r["dwgu"]))
        errs[f"dwd[{e}]"] = rel_fro(bf(host(out["dwd"][e]))[icols], bf(r["dwd"]))
        # columns i of dW_gate_up (each over H and both halves) and rows i of dW_down
        local[f"dwgu[{e}]"] = parity_stats(np.moveaxis(bf(host(out["dwgu"][e]))[:, :, icols], 2, 0),
                                           np.moveaxis(bf(r["dwgu"]), 2, 0), rows=len(icols))
        local[f"dwd[{e}]"] = parity_stats(bf(host(out["dwd"][e]))[icols], bf(r["dwd"]), rows=len(icols))
        if cfg.has_bias:
            errs[f"db1[{e}]"] = rel_fro(bf(host(out["db1"][e]))[:, icols], bf(r["db1"]))
            errs[f"db2[{e}]"] = rel_fro(bf(host(out["db2"][e])), bf(r["db2"]))
    empty = np.nonzero(cnt == 0)[0]
    for e in empty:
        assert not out["dwgu"][e].float().abs().sum().item() and not out["dwd"][e].float().abs().sum().item()
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    print(name, {k: {a: (f"{b:.2e}" if isinstance(b, float) else b) for a, b in v.items()}
                 for k, v in local.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    for k, st in local.items():
        assert_parity(k, st, tol=TOL)


def test_moe_stages_in_order_equal_one_call():
    """The per-stage entry point: stages 0..NUM_STAGES-1 run in order on a fresh
    workspace produce what one full call produces (bitwise for every output with
    a fixed summation order; the bias sums use atomics).  The last two cases have
    enough Phase-3 tiles (one to eight rounds over the CUs) for a full call to run
    the gathers and Phases 2 and 4 on the library's second stream."""
    cases = {**{n: SMALL[n] for n in ("medium_s", "fine_s", "fine_h256")},
             "medium_2s": S.scaled(S.MEDIUM, T=4096, H=1024, I=704, E=8, K=4, B=256),
             "fine_2s": S.scaled(S.FINE, T=4096, H=512, I=256, E=32, K=4, B=128)}
    for name, cfg in cases.items():
        g1 = gpu_problem(cfg)
        o1 = {k: v.clone() for k, v in g1["op"].run().items() if v is not None}
        g2 = gpu_problem(cfg)
        op = g2["op"]
        for s in range(op.NUM_STAGES):
            op.stage(s)
        torch.cuda.synchronize()
        o2 = op.out
        for k in ("dwgu", "dwd", "dx", "daff"):
            assert torch.equal(o1[k], o2[k]), (name, k)
        if cfg.has_bias:
            for k in ("db1", "db2"):
                assert rel_fro(bf(host(o2[k])), bf(host(o1[k]))) < 1e-5, (name, k)


# ----------------------------------------------------------------------------- supplied checkpoints
CKPT_CFGS = {"tiny_onH": S.TINY, "medium_s_onH": SMALL["medium_s"], "large_s_onI": SMALL["large_s"]}


def _exact_checkpoints(gp, p):
    """P1's optional checkpoints as the oracle computes them (fp64, rounded to
    bf16 where the recomputation rounds), laid out [N,I,B] / [N,B,H]; padding
    slots hold garbage, which the library must ignore."""
    cfg = gp["cfg"]
    N, B, I, H, E, T = gp["N"], cfg.B, cfg.I, cfg.H, cfg.E, cfg.T
    rng = np.random.default_rng(12)
    tpid = host(gp["tpid"]).reshape(N, B)
    pad = (tpid < 0) | (tpid >= T)                        # [N,B]
    b2e = host(gp["b2e"])
    a = np.where(pad, 0.0, gp["aff"].reshape(T, E)[np.where(pad, 0, tpid), b2e[:, None]]).astype(np.float32)
    ga = rng.integers(0, 1 << 16, (N, I, B), dtype=np.uint16)
    inter = rng.integers(0, 1 << 16, (N, I, B), dtype=np.uint16)
    for b in range(N):
        d = oracle.moe_block_detail(p, b)
        ga[b][:, ~pad[b]] = d["ga"].T[:, ~pad[b]]
        inter[b][:, ~pad[b]] = d["inter"].T[:, ~pad[b]]

    def to_bf16(x32):                                     # fp32 -> bf16 bits, nearest even
        return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)

    inter_f = (inter.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):   # padding slots hold garbage, replaced below
        scaled = to_bf16(inter_f * a[:, None, :])        # bf16(fp32(a * intermediate))
    scaled[np.broadcast_to(pad[:, None, :], scaled.shape)] = 0x7fc0
    dyf = (host(gp["t"]["dy"]).astype(np.uint32) << 16).view(np.float32)
    ady = to_bf16(dyf[np.where(pad, 0, tpid)] * a[:, :, None])   # bf16(fp32(a * dY[token])), [N,B,H]
    ady[pad] = rng.integers(0, 1 << 16, (int(pad.sum()), H), dtype=np.uint16)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return dict(gate_act_checkpoint_T=dev(ga), intermediate_checkpoint_T=dev(inter),
                scaled_intermediate_checkpoint_T=dev(scaled), down_proj_act_checkpoint=dev(ady))


@pytest.mark.parametrize("name", list(CKPT_CFGS))
def test_moe_supplied_checkpoints(name):
    """P1's optional checkpoints (silu(gate), the intermediate, and the scaled
    intermediate under the affinity on I or a*dY under the affinity on H) read
    in place of the recomputation: the gradients keep their parity with the
    oracle, and the operands built from the checkpoints are the oracle's bit
    for bit (recomputed on the GPU, the intermediate may differ in a rare
    bf16 rounding of silu)."""
    import mxfp8_grouped_gemm_amd as mx
    cfg = CKPT_CFGS[name]
    gp = gpu_problem(cfg)
    base = {k: v.clone() for k, v in gp["op"].run().items() if v is not None}
    p, ex = oracle_problem(gp)
    ck = _exact_checkpoints(gp, p)
    if cfg.affinity_on:
        del ck["down_proj_act_checkpoint"]
    else:
        del ck["scaled_intermediate_checkpoint_T"]
    t = gp["t"]
    gu_c, gu_s, d_c, d_s = gp["wq"]
    E, H, I = cfg.E, cfg.H, cfg.I
    op = mx.MoeBwd(t["hidden"], torch.from_numpy(gp["aff"]).cuda(), gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32),
                   d_c.view(E, I, H), d_s.view(E, I, H // 32), gp["tpid"], gp["b2e"], t["dy"], cfg.B, t["ckpt"],
                   down_proj_bias=t["b2"], affinity_on=cfg.affinity_on, **ck)
    out = op.run()
    torch.cuda.synchronize()
    ref = oracle.moe_bwd(p)
    _check_outputs(cfg, out, ref)
    for k in base:
        assert rel_fro(bf(host(out[k])), bf(host(base[k]))) <= 1e-3, k
    ws = op.workspace.cpu().numpy()
    L = op.layout
    P = gp["N"] * cfg.B
    c, s = oracle.moe_token_operand(p, oracle.TOK_INTER)
    assert np.array_equal(stage_major_to_rows(ws[L["inter_tok_codes"]:L["inter_tok_codes"] + I * P], I, P),
                          c.reshape(I, P))
    assert np.array_equal(pairs_to_rows(ws[L["inter_tok_scales"]:L["inter_tok_scales"] + I * P // 32], I, P),
                          s.reshape(I, P // 32))
    c, s = oracle.moe_token_operand(p, oracle.TOK_GY)
    assert np.array_equal(stage_major_to_rows(ws[L["gy_tok_codes"]:L["gy_tok_codes"] + H * P], H, P),
                          c.reshape(H, P))


def test_moe_checkpoints_rejected_with_the_wrong_affinity_placement():
    import mxfp8_grouped_gemm_amd as mx
    gp = gpu_problem(S.TINY)                       # affinity on H
    cfg = S.TINY
    bad = torch.zeros((gp["N"], cfg.I, cfg.B), dtype=torch.bfloat16, device="cuda")
    t = gp["t"]
    gu_c, gu_s, d_c, d_s = gp["wq"]
    E, H, I = cfg.E, cfg.H, cfg.I
    op = mx.MoeBwd(t["hidden"], torch.from_numpy(gp["aff"]).cuda(), gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32),
                   d_c.view(E, I, H), d_s.view(E, I, H // 32), gp["tpid"], gp["b2e"], t["dy"], cfg.B, t["ckpt"],
                   affinity_on=0, scaled_intermediate_checkpoint_T=bad)
    with pytest.raises(mx.MxError):
        op.run()


# ----------------------------------------------------------------------------- valid-token count
def _run_with_count(gp, n):
    import mxfp8_grouped_gemm_amd as mx
    cfg = gp["cfg"]
    t = gp["t"]
    gu_c, gu_s, d_c, d_s = gp["wq"]
    E, H, I = cfg.E, cfg.H, cfg.I
    nv = torch.tensor([n], dtype=torch.int32, device="cuda")
    op = mx.MoeBwd(t["hidden"], torch.from_numpy(gp["aff"]).cuda(), gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32),
                   d_c.view(E, I, H), d_s.view(E, I, H // 32), gp["tpid"], gp["b2e"], t["dy"], cfg.B, t["ckpt"],
                   down_proj_bias=t["b2"], affinity_on=cfg.affinity_on, num_valid_tokens=nv)
    out = op.run()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,counts", [("single_expert_dense", (200, 0, 300, 1000)), ("medium_s", (256, 1))])
def test_moe_num_valid_tokens(name, counts):
    """P1's num_valid_tokens: only the leading rows are real tokens (a count
    above T means T).  The oracle is given the same routing with the slots of
    tokens at or past the count made padding; those tokens' dX rows and d(a)
    entries must be exactly 0.  single_expert_dense is E = 1 with every token
    routed to expert 0 in order (the identity block layout)."""
    import dataclasses
    cfg = S.scaled(S.TINY, T=300, E=1, K=1) if name == "single_expert_dense" else SMALL[name]
    gp = gpu_problem(cfg)
    p, ex = oracle_problem(gp)
    for n in counts:
        out = _run_with_count(gp, n)
        nv = max(0, min(n, cfg.T))
        tp = np.where(p.tpid >= nv, -1, p.tpid).astype(np.int32)
        ref = oracle.moe_bwd(dataclasses.replace(p, tpid=tp))
        print(name, "count", n, flush=True)
        # the zeros this test owns are checked below; masking the routing can also
        # leave a chance exact zero in the oracle's dW (a cancelling sum, e.g.
        # dW_down[7][178][201] of medium_s at count 256) that fp32 order need not hit
        _check_outputs(cfg, out, ref, unrouted_zero=False)
        dx = host(out["dx"]).reshape(cfg.T, cfg.H)
        da = host(out["daff"]).reshape(cfg.T, cfg.E)
        assert not dx[nv:].any() and not da[nv:].any()


# ----------------------------------------------------------------------------- varlen-K routing
@pytest.mark.parametrize("name", ["tiny", "medium_s"])
def test_moe_dropped_selections(name):
    """Page 3's varlen-K routing: tokens activate between 0 and K experts
    (negative ids in the top-k list are dropped selections).  The routing
    blocks match the oracle's bit for bit, the gradients keep parity, and a
    token with no expert gets a zero dX row and zero d(a)."""
    import dataclasses
    import mxfp8_grouped_gemm_amd as mx
    cfg = SMALL[name]
    gp = gpu_problem(cfg)
    rng = np.random.default_rng(21)
    topk = gp["topk"].copy()
    topk[rng.random(topk.shape) < 0.3] = -1
    topk[3] = -1                                          # a token with no expert at all
    N = gp["N"]
    tpid, b2e = mx.moe_build_blocks(torch.from_numpy(topk).cuda(), cfg.E, cfg.B, N)
    rt, rb = oracle.build_blocks(topk, cfg.E, cfg.B, N)
    assert np.array_equal(host(tpid), rt) and np.array_equal(host(b2e), rb)
    t = gp["t"]
    gu_c, gu_s, d_c, d_s = gp["wq"]
    E, H, I = cfg.E, cfg.H, cfg.I
    op = mx.MoeBwd(t["hidden"], torch.from_numpy(gp["aff"]).cuda(), gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32),
                   d_c.view(E, I, H), d_s.view(E, I, H // 32), tpid, b2e, t["dy"], cfg.B, t["ckpt"],
                   down_proj_bias=t["b2"], affinity_on=cfg.affinity_on)
    out = op.run()
    torch.cuda.synchronize()
    p, _ = oracle_problem(gp)
    ref = oracle.moe_bwd(dataclasses.replace(p, tpid=rt, b2e=rb))
    _check_outputs(cfg, out, ref, unrouted_zero=False)
    assert not host(out["dx"]).reshape(cfg.T, H)[3].any()
    da = host(out["daff"]).reshape(cfg.T, E)
    assert not da[3].any()
    routed = np.zeros((cfg.T, E), bool)
    for tt in range(cfg.T):
        for e in topk[tt]:
            if e >= 0:
                routed[tt, e] = True
    assert not da[~routed].any()                          # dropped pairs get no affinity gradient


# ----------------------------------------------------------------------------- accumulation
@pytest.mark.parametrize("name", ["fine_s", "large_s"])
def test_moe_accumulate(name):
    """P1's accumulation flag (reading: add into the gradients).  Every output
    starts from seeded random bf16 values; one call must give bf16(prior + g)
    and a second call, on top of that, the oracle's accumulation of g onto its
    own first result.  Pairs without a slot keep the prior bit for bit."""
    import dataclasses
    import mxfp8_grouped_gemm_amd as mx
    cfg = SMALL[name]
    gp = gpu_problem(cfg)
    p, _ = oracle_problem(gp)
    base = oracle.moe_bwd(p)
    keys = ["dx", "daff", "dwgu", "dwd"] + (["db1", "db2"] if cfg.has_bias else [])
    rng = np.random.default_rng(61)
    prior = {}
    for k in keys:
        scale = float(np.abs(bf(base[k])).max())
        x = torch.from_numpy(rng.standard_normal(base[k].shape)).float() * scale
        prior[k] = S.bf16_bits(x.to(torch.bfloat16))
    t = gp["t"]
    gu_c, gu_s, d_c, d_s = gp["wq"]
    E, H, I = cfg.E, cfg.H, cfg.I
    op = mx.MoeBwd(t["hidden"], torch.from_numpy(gp["aff"]).cuda(), gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32),
                   d_c.view(E, I, H), d_s.view(E, I, H // 32), gp["tpid"], gp["b2e"], t["dy"], cfg.B, t["ckpt"],
                   down_proj_bias=t["b2"], affinity_on=cfg.affinity_on, accumulate=True)
    for k in keys:
        assert not op.out[k].float().abs().sum().item()          # allocated zeroed
        op.out[k].view(torch.int16).copy_(torch.from_numpy(prior[k].view(np.int16)).view(op.out[k].shape))
    pa = dataclasses.replace(p, accumulate=1)
    ref1 = oracle.moe_bwd(pa, prior=prior)
    out = op.run()
    torch.cuda.synchronize()
    print(name, "first call", flush=True)
    _check_outputs(cfg, out, ref1, unrouted_zero=False)
    routed = np.zeros((cfg.T, E), bool)
    routed[np.arange(cfg.T)[:, None], gp["topk"]] = True
    da = host(out["daff"]).reshape(cfg.T, E)
    assert np.array_equal(da[~routed], prior["daff"].reshape(cfg.T, E)[~routed])
    ref2 = oracle.moe_bwd(pa, prior=ref1)
    out = op.run()
    torch.cuda.synchronize()
    print(name, "second call", flush=True)
    _check_outputs(cfg, out, ref2, unrouted_zero=False)
    # the flag must not leak into a later overwriting problem
    again = gp["op"].run()
    torch.cuda.synchronize()
    _check_outputs(cfg, again, base)


# ----------------------------------------------------------------------------- GeGLU
def _bound_op(gp, **kw):
    """A MoeBwd over a problem's device tensors with extra arguments."""
    import mxfp8_grouped_gemm_amd as mx
    cfg, t = gp["cfg"], gp["t"]
    gu_c, gu_s, d_c, d_s = gp["wq"]
    E, H, I = cfg.E, cfg.H, cfg.I
    return mx.MoeBwd(t["hidden"], torch.from_numpy(gp["aff"]).cuda(), gu_c.view(E, H, 2, I),
                     gu_s.view(E, H, 2, I // 32), d_c.view(E, I, H), d_s.view(E, I, H // 32), gp["tpid"], gp["b2e"],
                     t["dy"], cfg.B, t["ckpt"], down_proj_bias=t["b2"], affinity_on=cfg.affinity_on, **kw)


@pytest.mark.parametrize("name", ["tiny", "medium_s", "fine_s", "large_s"])
def test_moe_geglu(name):
    """[P3]'s other gated activation, GeGLU (gelu in its erf form): every
    gradient keeps parity with the oracle's GeGLU backward, the intermediate
    operand's codes agree almost everywhere (erfc in fp32 against fp64), and
    the result differs from the SwiGLU one."""
    import dataclasses
    cfg = SMALL[name]
    gp = gpu_problem(cfg)
    sw = {k: v.clone() for k, v in gp["op"].run().items() if v is not None}
    op = _bound_op(gp, activation=1)
    out = op.run()
    torch.cuda.synchronize()
    p, _ = oracle_problem(gp)
    ref = oracle.moe_bwd(dataclasses.replace(p, activation=oracle.GEGLU))
    _check_outputs(cfg, out, ref)
    assert not torch.equal(sw["dx"], out["dx"])
    P = gp["N"] * cfg.B
    c, _ = oracle.moe_token_operand(dataclasses.replace(p, activation=oracle.GEGLU), oracle.TOK_INTER)
    got = op.workspace.cpu().numpy()[op.layout["inter_tok_codes"]:op.layout["inter_tok_codes"] + cfg.I * P]
    assert np.mean(stage_major_to_rows(got, cfg.I, P) != c.reshape(cfg.I, P)) < 1e-3
