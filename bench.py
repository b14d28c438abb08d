#!/usr/bin/env python3
"""Benchmark of the MXFP8 MoE backward on one MI355X.

A step is one pass of the hot path over one batch of seeded synthetic input
already resident in HBM: the routing blocks from the top-k ids
(moe_build_blocks) and the whole backward (moe_bwd_mxfp8: dY quantisation,
token-axis gathers, Phase 1 with its fused epilogue, Phases 3, 2 and 4, bias
reductions, finalisation).  The workload is the largest single-GPU MoE
configuration (T=16384, H=4096, I=14336, E=8, top-2, B=1024, affinity on the
intermediate).  The metric counts algorithmic FLOPs only: 12*H*I per routed
(token, expert) pair.

Printed: one JSON line on stdout (progress goes to stderr).  Besides the step
throughput it carries the roofline of the dominant kernel (timed live with HIP
events on the library's stream), the dense MXFP8 backward (4096^3), the
quantiser throughput, the router backward that consumes d(affinity) (every mode
on the fine workload's 32768 x 128 top-8 router), the CPU oracle timed on a
bounded sample, the step one call at a time with warm and with cold caches
(median, p10, p90), the same for the tiny, medium and fine workloads, and the
engine clock read from sysfs with the peak fraction rescaled to it.

roofline.traffic is the dominant kernel's HBM bytes per launch from two
rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) scaled by the same counters on
a copy of known size; it is read from profiles/<kernel>_<workload>_traffic.txt
and reported only while the kernel sources still hash to the value recorded
there (null otherwise).  Those passes run this script with --kernel-only and
--copy-calibration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense MXFP8 / FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # HBM3E


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = os.path.join(ROOT, "mxfp8_grouped_gemm_amd", "csrc")


NOT_MOE_SOURCES = ("router.hip",)   # kernels no MoE-backward stage is built from


def sources_sha256():
    """Hash of the HIP sources the MoE-backward stages are built from (kernels,
    headers and the launch code), to tell whether counters taken earlier still
    describe the kernels being timed."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCES)):
        if name.endswith((".hip", ".hpp", ".cpp", ".h")) and name not in NOT_MOE_SOURCES:
            h.update(name.encode())
            with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch recorded for (kernel, workload), or None when there
    is no record or the sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("sources_sha256") != sources_sha256() or "traffic_bytes_per_launch" not in rec:
        return None
    return float(rec["traffic_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events_ms(fn, reps):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def step_distribution(fn, reps, cold, scratch=None):
    """Per-call durations of fn (HIP events around each call): median, p10 and
    p90 in ms.  cold: a 512 MiB buffer is written before each call (outside the
    events), which evicts the L2s and the 256 MB infinity cache."""
    import numpy as np
    import torch
    if cold and scratch is None:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        if cold:
            scratch.fill_(1)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": round(float(np.median(t)), 4), "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4), "reps": reps}


def gpu_sclk_mhz():
    """Current shader clock from sysfs (the starred pp_dpm_sclk level), or None."""
    import glob
    import re
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if "*" in line:
                    m = re.search(r"(\d+)\s*[Mm]hz", line)
                    if m:
                        return int(m.group(1))
        except OSError:
            pass
    return None


def stage_work(cfg, N):
    """Algorithmic FLOPs (MFMA stages) or bytes (HBM stages) of each stage."""
    T, H, I, E, K, B = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.B
    TK, P = T * K, N * B
    q = 1 + 1 / 32                      # bytes per quantised element (code + its share of a scale)
    return {
        # slot routing info (token, affinity, the (token, expert) -> slot map, block
        # extents and lists) and the zeroed per-slot d(a) bias term
        "setup": ("hbm", P * 20 + T * E * 8),
        # dY: bf16 in, codes + scales out; H % 128 == 0: W_down's and W_gate_up's scales
        # re-laid pair-major (read + write); otherwise Phase 1 reads bf16 values, so dY's
        # are written too and W_down's codes are read and their bf16 values written
        "quantize_dy": ("hbm", T * H * (2 + q) + E * H * 2 * I / 32 * 2
                        + (E * I * H / 32 * 2 if H % 128 == 0 else T * H * 2 + E * I * H * (q + 2))),
        "gather_quantize_x_dy": ("hbm", 2 * (TK * H * 2 + P * H * q)),
        "bias": ("hbm", 2 * TK * H * 2 if cfg.has_bias else 0),
        "phase1": ("mfma_bf16", 2 * TK * H * I),
        # per (pair, i): reads g, u and dS; writes dGU quantised along both axes and
        # the intermediate quantised
        "phase1_epilogue": ("hbm", TK * I * (4 + 4 + 5 * q)),
        "phase3": ("mfma", 4 * TK * H * I),
        "phase2": ("mfma", 4 * TK * H * I),
        "phase4": ("mfma", 2 * TK * H * I),
        # dX: each routed pair's fp32 row read, the token's bf16 row written; d(a)
        "finalize": ("hbm", TK * H * 4 + T * H * 2 + P * 4 * (1 + I // 32) + T * E * (4 + 2)),
    }


def roofline_of(kind, work, ms):
    if kind.startswith("mfma"):
        ach = work / (ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if kind == "mfma_bf16" else PEAK_FP8_TFLOPS
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    ach = work / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def build_problem(cfg, keep_w01=False):
    """Seeded synthetic inputs of cfg resident on the GPU, weights quantised by
    the library, routing blocks built, the backward operator bound."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    import synthetic as S

    dev = "cuda"
    topk, aff = S.routing(cfg)
    N = mx.moe_num_blocks(cfg.T, cfg.K, cfg.E, cfg.B)
    topk_d = torch.from_numpy(topk).to(dev)
    L = mx.lib()
    rb_ws = torch.empty(L.moe_build_blocks_workspace_size(cfg.E), dtype=torch.uint8, device=dev)
    tpid = torch.empty(N * cfg.B, dtype=torch.int32, device=dev)
    b2e = torch.empty(N, dtype=torch.int32, device=dev)
    mx.moe_build_blocks(topk_d, cfg.E, cfg.B, N, out=(tpid, b2e), workspace=rb_ws)
    t = S.moe_tensors(cfg, N, dev)
    E, H, I = cfg.E, cfg.H, cfg.I
    gu_c, gu_s = mx.mxfp8_quantize(t["w_gate_up"].view(E * H * 2, I), 1, mx.E4M3)
    d_c, d_s = mx.mxfp8_quantize(t["w_down"].view(E * I, H), 1, mx.E4M3)
    w01 = None
    if keep_w01:      # experts 0 and 1 for the CPU-baseline sample (generator output)
        w01 = {"gu": S.bf16_bits(t["w_gate_up"][:2]), "d": S.bf16_bits(t["w_down"][:2])}
    del t["w_gate_up"], t["w_down"]
    aff_d = torch.from_numpy(aff).to(dev)
    op = mx.MoeBwd(t["hidden"], aff_d, gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32), d_c.view(E, I, H),
                   d_s.view(E, I, H // 32), tpid, b2e, t["dy"], cfg.B, t["ckpt"], down_proj_bias=t["b2"],
                   affinity_on=cfg.affinity_on)
    return dict(op=op, N=N, topk=topk, aff=aff, topk_d=topk_d, tpid=tpid, b2e=b2e, rb_ws=rb_ws, t=t, w01=w01)


def run_moe(cfg, steps, warmup, profile_reps, keep_w01=False, distributions=True):
    import torch
    import mxfp8_grouped_gemm_amd as mx

    pb = build_problem(cfg, keep_w01)
    op, N, topk_d, tpid, b2e, rb_ws = pb["op"], pb["N"], pb["topk_d"], pb["tpid"], pb["b2e"], pb["rb_ws"]
    log(f"[bench] {cfg.name}: N={N} blocks, workspace {op.workspace.numel() / 2**30:.2f} GiB")

    def step():
        mx.moe_build_blocks(topk_d, cfg.E, cfg.B, N, out=(tpid, b2e), workspace=rb_ws)
        op.run()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({warmup} steps)")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / steps
    sclk = gpu_sclk_mhz()
    log(f"[bench] timed {steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s), sclk {sclk} MHz")
    # the step one at a time: warm caches, then cold (L2 and infinity cache evicted)
    timing = None
    if distributions:
        timing = {"warm": step_distribution(step, 20, False), "cold": step_distribution(step, 20, True)}
        log(f"[bench] per step: warm {timing['warm']}, cold {timing['cold']}")

    # per-stage durations, HIP events on the stream the library launches on
    work = stage_work(cfg, N)
    stages = {}
    for s, name in enumerate(op.STAGE_NAMES):
        if name == "bias" and not cfg.has_bias:
            continue
        stages[name] = _events_ms(lambda s=s: op.stage(s), profile_reps)
    stages["build_blocks"] = _events_ms(
        lambda: mx.moe_build_blocks(topk_d, cfg.E, cfg.B, N, out=(tpid, b2e), workspace=rb_ws), profile_reps)
    op.run()
    torch.cuda.synchronize()
    dom = max((k for k in stages if k in work), key=lambda k: stages[k])
    kind, w = work[dom]
    roof = roofline_of(kind, w, stages[dom])
    roof.update({"kernel": dom, "launch_ms": round(stages[dom], 4), "traffic": recorded_traffic(dom, cfg.name)})
    per_stage = {k: {"ms": round(v, 4), **({} if k not in work or not work[k][1] else
                                           {kk: vv for kk, vv in roofline_of(work[k][0], work[k][1], v).items()
                                            if kk in ("achieved", "unit", "frac")})}
                 for k, v in stages.items()}
    log(f"[bench] stages: " + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))
    return dict(ms=ms, wall=wall, roof=roof, stages=per_stage, N=N, topk=pb["topk"], aff=pb["aff"], tensors=pb["t"],
                w01=pb["w01"], timing=timing, sclk=sclk)


def run_other_configs(skip):
    """The other MoE workloads, each a full step (routing blocks + backward):
    warm and cold distributions; TFLOP/s from the cold median for the medium
    and fine workloads and from the warm one for tiny, which is launch-bound."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    import synthetic as S
    res = {}
    for name, cfg in S.MOE_CONFIGS.items():
        if cfg.name == skip:
            continue
        pb = build_problem(cfg)
        op, N, topk_d, tpid, b2e, rb_ws = pb["op"], pb["N"], pb["topk_d"], pb["tpid"], pb["b2e"], pb["rb_ws"]

        def step():
            mx.moe_build_blocks(topk_d, cfg.E, cfg.B, N, out=(tpid, b2e), workspace=rb_ws)
            op.run()

        for _ in range(5):
            step()
        reps = 200 if name == "tiny" else 20
        warm, cold = step_distribution(step, reps, False), step_distribution(step, reps, True)
        prim = "warm" if name == "tiny" else "cold"
        tf = cfg.flops / ({"warm": warm, "cold": cold}[prim]["median_ms"] * 1e9)
        res[name] = {"workload": cfg.name, "warm": warm, "cold": cold, "primary": prim,
                     "TFLOP/s": round(tf, 2), "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        log(f"[bench] {cfg.name}: warm {warm['median_ms']} ms, cold {cold['median_ms']} ms, {tf:.1f} TFLOP/s ({prim})")
        del pb, op
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def run_dense(reps):
    import torch
    import mxfp8_grouped_gemm_amd as mx
    import synthetic as S
    cfg = S.DENSE
    t = S.dense_tensors(cfg, "cuda")
    M, Nn, K = cfg.M, cfg.N, cfg.K
    ws = torch.empty(mx.lib().matmul_mxfp8_bwd_workspace_size(M, Nn, K), dtype=torch.uint8, device="cuda")
    out = (torch.empty((M, K), dtype=torch.bfloat16, device="cuda"),
           torch.empty((Nn, K), dtype=torch.bfloat16, device="cuda"))
    call = lambda: mx.matmul_mxfp8_bwd(t["dy"], t["w"], t["x"], workspace=ws, out=out)
    call()
    ms = _events_ms(call, reps)
    st = [_events_ms(lambda s=s: mx.matmul_mxfp8_bwd_stage(t["dy"], t["w"], t["x"], s, ws, out), reps)
          for s in range(4)]
    gemm_flops = 2 * M * Nn * K
    res = {"workload": cfg.name, "ms": round(ms, 4), "TFLOP/s": round(cfg.flops / ms / 1e9, 2),
           "frac_of_fp8_peak": round(cfg.flops / ms / 1e9 / PEAK_FP8_TFLOPS, 4),
           "dX_gemm": roofline_of("mfma", gemm_flops, st[2]) | {"ms": round(st[2], 4)},
           "dW_gemm": roofline_of("mfma", gemm_flops, st[3]) | {"ms": round(st[3], 4)},
           "quantize_N_ms": round(st[0], 4), "quantize_M_ms": round(st[1], 4)}
    x = S.normal_bf16((4096, 4096), 1.0, 0, 99, "cuda")
    qms = _events_ms(lambda: mx.mxfp8_quantize(x, 1, mx.E4M3), reps)
    qbytes = 4096 * 4096 * (2 + 1 + 1 / 32)
    res_q = {"shape": [4096, 4096], "axis": 1, "ms": round(qms, 5), **roofline_of("hbm", qbytes, qms)}
    return res, res_q


def run_router(reps):
    """The router backward on the fine workload's router (32768 tokens, 128
    experts, top-8): every mode, with the algorithmic bytes of one launch
    (selections and score gradients read, logits read where the mode needs
    them, every logit gradient written)."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    T, E, K = 32768, 128, 8
    gen = torch.Generator(device="cuda").manual_seed(7)
    logits = torch.randn((T, E), generator=gen, device="cuda", dtype=torch.float32) * 2.0
    idx = torch.topk(logits, K, dim=1).indices.to(torch.int32).contiguous()
    g = torch.randn((T, K), generator=gen, device="cuda", dtype=torch.float32)
    sel = torch.gather(logits, 1, idx.long())
    y = torch.softmax(sel, dim=1).contiguous()                     # forward scores, softmax over the top-k
    ps = torch.gather(torch.softmax(logits, dim=1), 1, idx.long())
    s = (ps / ps.sum(dim=1, keepdim=True)).contiguous()            # forward scores, renormalised top-k of the softmax
    res = {"workload": f"router_T{T}_E{E}_top{K}"}
    for name, mode, renorm, sc, lg, nbytes in (
            ("softmax_over_topk", mx.ROUTER_SOFTMAX_OVER_TOPK, False, y, None, T * (12 * K + 4 * E)),
            ("topk_over_softmax", mx.ROUTER_TOPK_OVER_SOFTMAX, False, None, logits, T * (8 * K + 8 * E)),
            ("topk_over_softmax_renorm", mx.ROUTER_TOPK_OVER_SOFTMAX, True, s, logits, T * (12 * K + 8 * E)),
            ("topk_scatter", mx.ROUTER_TOPK, False, None, None, T * (8 * K + 4 * E))):
        out = torch.empty((T, E), dtype=torch.float32, device="cuda")
        call = lambda: mx.moe_router_bwd(mode, idx, dscores=g, topk_scores=sc, logits=lg, num_experts=E,
                                         renorm=renorm, out=out)
        call()
        ms = _events_ms(call, reps)
        res[name] = {"ms": round(ms, 5), **roofline_of("hbm", nbytes, ms)}
    return res


def cpu_baseline(cfg, moe, nthreads, n_tokens, n_cols):
    """The oracle (as it stands) on a bounded sample of the same workload: whole
    dX rows and d(a) of n_tokens tokens routed only to experts {0,1} (Phases 1
    and 3 with the epilogue), and n_cols intermediate columns of expert 0's
    weight gradients (Phases 2 and 4).  Weights of experts 0 and 1 are
    quantised by the oracle itself (input preparation, not timed)."""
    import numpy as np
    import oracle
    import synthetic as S
    T, H, I, E, B = cfg.T, cfg.H, cfg.I, cfg.E, cfg.B
    N = moe["N"]
    t = moe["tensors"]
    bits = {k: (None if v is None else S.bf16_bits(v)) for k, v in t.items()}
    tpid, b2e = oracle.build_blocks(moe["topk"], E, B, N)
    topk = moe["topk"]
    wgu_c = np.zeros((E, H, 2, I), np.uint8)
    wgu_s = np.zeros((E, H, 2, I // 32), np.uint8)
    wd_c = np.zeros((E, I, H), np.uint8)
    wd_s = np.zeros((E, I, H // 32), np.uint8)
    # bf16 weights of experts 0 and 1 as the generator made them, quantised by the oracle
    from concurrent.futures import ThreadPoolExecutor

    def q_rows(x, rows):
        return oracle.quantize(np.ascontiguousarray(x[rows]), 1, oracle.E4M3)

    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        for e in (0, 1):
            gu = moe["w01"]["gu"][e].reshape(H * 2, I)
            dd = moe["w01"]["d"][e].reshape(I, H)
            for src, dst_c, dst_s in ((gu, wgu_c[e].reshape(H * 2, I), wgu_s[e].reshape(H * 2, I // 32)),
                                      (dd, wd_c[e], wd_s[e])):
                chunks = np.array_split(np.arange(src.shape[0]), nthreads)
                for rows, (c, s) in zip(chunks, ex.map(lambda r, src=src: q_rows(src, r), chunks)):
                    dst_c[rows], dst_s[rows] = c, s
    p = oracle.MoeProblem(T=T, H=H, I=I, E=E, N=N, B=B, hidden=bits["hidden"], aff=moe["aff"], wgu_codes=wgu_c,
                          wgu_scales=wgu_s, wd_codes=wd_c, wd_scales=wd_s, tpid=tpid, b2e=b2e, dy=bits["dy"],
                          ckpt=bits["ckpt"], b2=bits["b2"], affinity_on=cfg.affinity_on,
                          has_bias=int(cfg.has_bias), nthreads=nthreads)
    only01 = np.nonzero(np.all(np.isin(topk, [0, 1]), axis=1))[0][:n_tokens].astype(np.int32)
    cols = np.arange(n_cols, dtype=np.int32) * (I // n_cols)
    slots_e0 = int(np.count_nonzero((tpid >= 0) & (np.repeat(b2e, B) == 0)))
    t0 = time.perf_counter()
    oracle.moe_token_rows(p, only01)
    t1 = time.perf_counter()
    oracle.moe_expert_cols(p, 0, cols)
    t2 = time.perf_counter()
    flops = only01.size * cfg.K * 6 * H * I + n_cols * 6 * H * slots_e0
    secs = t2 - t0
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": (f"{cfg.name}: dX rows + d(affinity) of {only01.size} tokens (Phases 1+3, {t1 - t0:.1f} s) "
                       f"and {n_cols} intermediate columns of expert 0's dW (Phases 2+4, {slots_e0} slots, "
                       f"{t2 - t1:.1f} s); {flops / 1e9:.1f} GFLOP in {secs:.1f} s")}


def kernel_only(cfg, stage_name, reps):
    """Set the workload up, run the backward once, then launch one stage reps
    times (the program rocprofv3 --pmc wraps for that stage's counters)."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    op = build_problem(cfg)["op"]
    op.run()
    torch.cuda.synchronize()
    s = op.STAGE_NAMES.index(stage_name)
    for _ in range(reps):
        op.stage(s)
    torch.cuda.synchronize()
    log(f"[bench] kernel-only: {stage_name} x{reps} on {cfg.name} (library {mx.version()})")


def copy_calibration(nbytes):
    """One device-to-device copy of nbytes by a plain copy kernel (torch's
    elementwise copy), after a warm-up copy: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {nbytes} bytes read and written")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="large", choices=["tiny", "medium", "large", "fine"])
    ap.add_argument("--profile-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--cpu-cols", type=int, default=128)
    ap.add_argument("--kernel-only", metavar="STAGE", help="set up, then launch one stage (for rocprofv3 --pmc)")
    ap.add_argument("--copy-calibration", type=int, metavar="BYTES", help="one copy of BYTES (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic as S
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cfg = S.MOE_CONFIGS[args.workload]
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.kernel_only:
        kernel_only(cfg, args.kernel_only, max(1, args.steps))
        return
    moe = run_moe(cfg, args.steps, args.warmup, args.profile_reps, keep_w01=not args.no_cpu_baseline,
                  distributions=not args.no_extra)
    value = cfg.flops / moe["ms"] / 1e9
    out = {
        "metric": "MoE backward TFLOP/s (1 MI355X) + % of MXFP8 MFMA peak; quantize GB/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(moe["ms"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "top_k": cfg.K,
                   "block_size": cfg.B, "affinity_on": "I" if cfg.affinity_on else "H", "bias": cfg.has_bias,
                   "seed": cfg.seed, "parallelism": "single-gpu"},
        "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4),
        "roofline": moe["roof"],
        "stages": moe["stages"],
        "step_timing": moe["timing"],
        # the 5.0 PFLOP/s peak is quoted at the 2.4 GHz peak engine clock
        "sclk_mhz": moe["sclk"],
        "frac_of_fp8_peak_at_sclk": (round(value / (PEAK_FP8_TFLOPS * moe["sclk"] / 2400.0), 4)
                                     if moe["sclk"] else None),
    }
    if not args.no_extra:
        dense, quant = run_dense(args.profile_reps + 5)
        out["dense"] = dense
        out["quantize"] = quant
        log(f"[bench] dense: {dense['TFLOP/s']} TFLOP/s; quantize {quant['achieved']} GB/s")
        out["router_bwd"] = run_router(args.profile_reps + 5)
        log("[bench] router backward: " + ", ".join(f"{k} {v['ms']} ms" for k, v in out["router_bwd"].items()
                                                     if isinstance(v, dict)))
        out["other_workloads"] = run_other_configs(cfg.name)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample) ...")
        out["cpu_baseline"] = cpu_baseline(cfg, moe, args.cpu_threads, args.cpu_tokens, args.cpu_cols)
        log(f"[bench] cpu baseline: {out['cpu_baseline']['sample']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
