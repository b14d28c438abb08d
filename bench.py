#!/usr/bin/env python3
"""Benchmark of the MXFP8 MoE backward on one MI355X.

A step is one pass of the hot path over one batch of seeded synthetic input
already resident in HBM: the routing blocks from the top-k ids
(moe_build_blocks) and the whole backward (moe_bwd_mxfp8: dY quantisation,
token-axis gathers, Phase 1 and its SwiGLU-backward epilogue kernel, Phases 3, 2 and 4, bias
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
    # stages that another one does (their own launch is then empty): the bias
    # reductions inside the dY gather (a bias, H % 128 == 0), the epilogue inside
    # Phase 1's kernel (H % 128 == 0, H <= 2048, I <= 512; no optional checkpoints here)
    bias_fused = cfg.has_bias and H % 128 == 0
    epi_fused = H % 128 == 0 and H <= 2048 and I <= 512
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
        "bias": ("hbm", 2 * TK * H * 2 if cfg.has_bias and not bias_fused else 0),
        "phase1": ("mfma_bf16", 2 * TK * H * I),
        # per (pair, i): reads g, u and dS; writes dGU quantised along both axes and
        # the intermediate quantised
        "phase1_epilogue": ("hbm", 0 if epi_fused else TK * I * (4 + 4 + 5 * q)),
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
        r = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
             "frac": round(ach / peak, 4)}
        if kind == "mfma_bf16":   # the same MX product, also against the MXFP8 peak
            r["frac_of_fp8_peak"] = round(ach / PEAK_FP8_TFLOPS, 4)
        return r
    ach = work / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def build_problem(cfg, keep_w01=False, keep_w_all=False):
    """Seeded synthetic inputs of cfg resident on the GPU, weights quantised by
    the library, routing blocks built, the backward operator bound.  keep_w01 /
    keep_w_all: host copies of the bf16 weights of experts 0 and 1 / of every
    expert, for the oracle's sample (the generator's output, before the library
    quantises it)."""
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
    if keep_w01 or keep_w_all:      # for the CPU-baseline sample (generator output)
        n = E if keep_w_all else 2
        w01 = {"gu": S.bf16_bits(t["w_gate_up"][:n]), "d": S.bf16_bits(t["w_down"][:n])}
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

    stages, per_stage, dom = time_stages(cfg, pb, profile_reps)
    kind, w = stage_work(cfg, N)[dom]
    roof = roofline_of(kind, w, stages[dom])
    roof.update({"kernel": dom, "launch_ms": round(stages[dom], 4), "traffic": recorded_traffic(dom, cfg.name)})
    return dict(ms=ms, wall=wall, roof=roof, stages=per_stage, N=N, topk=pb["topk"], aff=pb["aff"], tensors=pb["t"],
                w01=pb["w01"], timing=timing, sclk=sclk)


def time_stages(cfg, pb, reps):
    """Per-stage durations (HIP events on the stream the library launches on),
    each with its roofline figure; also the stage with the longest launch."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    op, N, topk_d, tpid, b2e, rb_ws = pb["op"], pb["N"], pb["topk_d"], pb["tpid"], pb["b2e"], pb["rb_ws"]
    work = stage_work(cfg, N)
    stages = {}
    for s, name in enumerate(op.STAGE_NAMES):
        if name == "bias" and not cfg.has_bias:
            continue
        stages[name] = _events_ms(lambda s=s: op.stage(s), reps)
    stages["build_blocks"] = _events_ms(
        lambda: mx.moe_build_blocks(topk_d, cfg.E, cfg.B, N, out=(tpid, b2e), workspace=rb_ws), reps)
    op.run()
    torch.cuda.synchronize()
    dom = max((k for k in stages if k in work), key=lambda k: stages[k])
    per_stage = {k: {"ms": round(v, 4), **({} if k not in work or not work[k][1] else
                                           {kk: vv for kk, vv in roofline_of(work[k][0], work[k][1], v).items()
                                            if kk in ("achieved", "unit", "frac")})}
                 for k, v in stages.items()}
    log(f"[bench] {cfg.name} stages: " + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))
    return stages, per_stage, dom


def run_other_configs(skip, cpu_threads=0, profile_reps=5):
    """The other MoE workloads, each a full step (routing blocks + backward):
    warm and cold distributions, per-stage times, and (cpu_threads > 0) the
    oracle timed on a bounded sample of the same workload.  TFLOP/s from the
    cold median for the medium and fine workloads and from the warm one for
    tiny, which is launch-bound."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    import synthetic as S
    res, cpu = {}, {}
    for name, cfg in S.MOE_CONFIGS.items():
        if cfg.name == skip:
            continue
        pb = build_problem(cfg, keep_w_all=cpu_threads > 0)
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
        _, per_stage, dom = time_stages(cfg, pb, profile_reps)
        res[name] = {"workload": cfg.name, "warm": warm, "cold": cold, "primary": prim,
                     "TFLOP/s": round(tf, 2), "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                     "stages": per_stage, "longest_stage": dom}
        log(f"[bench] {cfg.name}: warm {warm['median_ms']} ms, cold {cold['median_ms']} ms, {tf:.1f} TFLOP/s ({prim})")
        if cpu_threads > 0:
            host = dict(N=N, topk=pb["topk"], aff=pb["aff"], tensors=pb["t"], w01=pb["w01"])
            cpu[name] = oracle_sample(cfg, host, cpu_threads, all_experts=True,
                                      **({"full": True} if name == "tiny" else {"n_tokens": 512, "n_cols": 128}))
            if name == "tiny":     # the whole tiny backward on one thread as well
                cpu[name]["single_thread"] = oracle_sample(cfg, host, 1, all_experts=True, full=True)
            log(f"[bench] cpu baseline {name}: {cpu[name]['sample']}")
        del pb, op
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res, cpu


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
    qout = mx.mxfp8_quantize(x, 1, mx.E4M3)   # outputs allocated once, outside the timed calls
    qms = _events_ms(lambda: mx.mxfp8_quantize(x, 1, mx.E4M3, out=qout), reps)
    qbytes = 4096 * 4096 * (2 + 1 + 1 / 32)
    res_q = {"shape": [4096, 4096], "axis": 1, "ms": round(qms, 5), **roofline_of("hbm", qbytes, qms)}
    # the same on an input larger than the 256 MB infinity cache (512 MiB), so
    # back-to-back calls read it from HBM; start and drain are a small part of it
    xl = S.normal_bf16((16384, 16384), 1.0, 0, 98, "cuda")
    qlout = mx.mxfp8_quantize(xl, 1, mx.E4M3)
    qlms = _events_ms(lambda: mx.mxfp8_quantize(xl, 1, mx.E4M3, out=qlout), reps)
    res_q["larger"] = {"shape": [16384, 16384], "axis": 1, "ms": round(qlms, 5),
                       **roofline_of("hbm", 16384 * 16384 * (2 + 1 + 1 / 32), qlms)}
    del xl, qlout
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


def host_cpu():
    """The host the oracle runs on: logical CPUs of the machine, those this
    process may run on, the thread share the box grants a one-GPU job
    (OMP_NUM_THREADS there), and the CPU model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or None
    return {"cpu_model": model, "host_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
            "thread_share": share}


def oracle_threads():
    """Threads for the oracle: every CPU this process may run on, capped at the
    box's per-GPU thread share when one is set."""
    h = host_cpu()
    n = h["affinity_cpus"] or 1
    return min(n, h["thread_share"]) if h["thread_share"] else n


def oracle_sample(cfg, moe, nthreads, n_tokens=0, n_cols=0, all_experts=False, full=False):
    """The oracle (as it stands, never tuned for timing) on the same workload:
    full=True the whole backward; otherwise a bounded sample: whole dX rows and
    d(a) of n_tokens tokens (Phases 1 and 3 with the epilogue) and n_cols
    intermediate columns of one expert's weight gradients (Phases 2 and 4).
    With all_experts every expert's weights are quantised by the oracle (input
    preparation, not timed); otherwise only experts 0 and 1, and the tokens are
    those routed to no other expert.  The rate counts the algorithmic FLOPs of
    the sample (12*H*I per routed pair of the rows, 6*H per slot and column)."""
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
    from concurrent.futures import ThreadPoolExecutor

    def q_rows(x, rows):
        return oracle.quantize(np.ascontiguousarray(x[rows]), 1, oracle.E4M3)

    nq = moe["w01"]["gu"].shape[0]
    with ThreadPoolExecutor(max_workers=max(1, nthreads)) as ex:
        for e in range(nq):
            gu = moe["w01"]["gu"][e].reshape(H * 2, I)
            dd = moe["w01"]["d"][e].reshape(I, H)
            for src, dst_c, dst_s in ((gu, wgu_c[e].reshape(H * 2, I), wgu_s[e].reshape(H * 2, I // 32)),
                                      (dd, wd_c[e], wd_s[e])):
                chunks = np.array_split(np.arange(src.shape[0]), max(1, nthreads))
                for rows, (c, s) in zip(chunks, ex.map(lambda r, src=src: q_rows(src, r), chunks)):
                    dst_c[rows], dst_s[rows] = c, s
    p = oracle.MoeProblem(T=T, H=H, I=I, E=E, N=N, B=B, hidden=bits["hidden"], aff=moe["aff"], wgu_codes=wgu_c,
                          wgu_scales=wgu_s, wd_codes=wd_c, wd_scales=wd_s, tpid=tpid, b2e=b2e, dy=bits["dy"],
                          ckpt=bits["ckpt"], b2=bits["b2"], affinity_on=cfg.affinity_on,
                          has_bias=int(cfg.has_bias), nthreads=nthreads)
    if full:
        t0 = time.perf_counter()
        oracle.moe_bwd(p)
        secs = time.perf_counter() - t0
        flops = cfg.flops
        desc = f"{cfg.name}: the whole backward, {flops / 1e9:.2f} GFLOP in {secs:.2f} s on {nthreads} thread(s)"
    else:
        if all_experts:
            toks = np.arange(min(n_tokens, T), dtype=np.int32)
        else:
            toks = np.nonzero(np.all(np.isin(topk, [0, 1]), axis=1))[0][:n_tokens].astype(np.int32)
        cnt = np.bincount(topk[topk >= 0].ravel(), minlength=E)
        e_cols = int(np.argmax(cnt)) if all_experts else 0
        cols = np.arange(n_cols, dtype=np.int32) * (I // n_cols)
        slots = int(np.count_nonzero((tpid >= 0) & (np.repeat(b2e, B) == e_cols)))
        pairs = int(np.count_nonzero(topk[toks] >= 0))
        t0 = time.perf_counter()
        oracle.moe_token_rows(p, toks)
        t1 = time.perf_counter()
        oracle.moe_expert_cols(p, e_cols, cols)
        t2 = time.perf_counter()
        flops = pairs * 6 * H * I + n_cols * 6 * H * slots
        secs = t2 - t0
        desc = (f"{cfg.name}: dX rows + d(affinity) of {toks.size} tokens ({pairs} routed pairs; Phases 1+3, "
                f"{t1 - t0:.1f} s) and {n_cols} intermediate columns of expert {e_cols}'s dW (Phases 2+4, {slots} "
                f"slots, {t2 - t1:.1f} s); {flops / 1e9:.1f} GFLOP in {secs:.1f} s on {nthreads} thread(s)")
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "seconds": round(secs, 3), "sample": desc}


def oracle_dense_sample(nthreads, n_rows):
    """The oracle's dense backward (4096^3) on n_rows rows of dX and of dW: the
    whole-operand quantisations it needs plus 4*n_rows*4096*4096 FLOPs."""
    import numpy as np
    import oracle
    import synthetic as S
    cfg = S.DENSE
    d = S.dense_tensors(cfg, "cpu")
    dy, w, x = (S.bf16_bits(d[k]) for k in ("dy", "w", "x"))
    rows = np.arange(n_rows, dtype=np.int64) * (cfg.M // n_rows)
    t0 = time.perf_counter()
    oracle.dense_bwd(dy, w, x, dx_rows=rows, dw_rows=rows, nthreads=nthreads)
    secs = time.perf_counter() - t0
    flops = 2 * 2 * n_rows * cfg.N * cfg.K
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "seconds": round(secs, 3),
            "sample": f"{cfg.name}: {n_rows} rows of dX and of dW (with the quantisation of all three operands), "
                      f"{flops / 1e9:.2f} GFLOP in {secs:.2f} s on {nthreads} thread(s)"}


def kernel_only(cfg, stage_names, reps):
    """Set the workload up, run the backward once, then launch each of the
    comma-separated stages reps times (the program rocprofv3 --pmc wraps for
    those stages' counters)."""
    import torch
    import mxfp8_grouped_gemm_amd as mx
    op = build_problem(cfg)["op"]
    op.run()
    torch.cuda.synchronize()
    for name in stage_names.split(","):
        s = op.STAGE_NAMES.index(name)
        for _ in range(reps):
            op.stage(s)
        torch.cuda.synchronize()
        log(f"[bench] kernel-only: {name} x{reps} on {cfg.name} (library {mx.version()})")


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
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (0: every CPU this process may use, capped at the box's thread share)")
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--cpu-cols", type=int, default=128)
    ap.add_argument("--kernel-only", metavar="STAGES",
                    help="set up, then launch the comma-separated stages (for rocprofv3 --pmc)")
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
        log(f"[bench] dense: {dense['TFLOP/s']} TFLOP/s; quantize {quant['achieved']} GB/s "
            f"([16384, 16384]: {quant['larger']['achieved']} GB/s)")
        out["router_bwd"] = run_router(args.profile_reps + 5)
        log("[bench] router backward: " + ", ".join(f"{k} {v['ms']} ms" for k, v in out["router_bwd"].items()
                                                     if isinstance(v, dict)))
    nthreads = args.cpu_threads or oracle_threads()
    others_cpu = {}
    if not args.no_extra:
        out["other_workloads"], others_cpu = run_other_configs(
            cfg.name, 0 if args.no_cpu_baseline else nthreads, args.profile_reps)
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle on a bounded sample, {nthreads} threads) ...")
        cb = oracle_sample(cfg, moe, nthreads, args.cpu_tokens, args.cpu_cols)
        cb.update(host_cpu())
        if not args.no_extra:
            dense_st = oracle_dense_sample(1, 32)
            dense_mt = oracle_dense_sample(nthreads, 256)
            dense_mt["single_thread"] = dense_st
            cb["other_workloads"] = {**others_cpu, "dense": dense_mt}
        out["cpu_baseline"] = cb
        log(f"[bench] cpu baseline: {cb['sample']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
