"""Shared set-up of MoE problems for the GPU tests, the smoke check and the benchmark.

One problem = seeded synthetic inputs on the device, routing blocks built by the
library, weights quantised by the library (GPU side), and -- for tests -- the
same inputs copied to the host with the oracle's own routing and weight codes.
"""
from __future__ import annotations

import numpy as np
import torch

import synthetic as S


def gpu_problem(cfg: S.MoeConfig, N: int = None, device="cuda"):
    import mxfp8_grouped_gemm_amd as mx
    topk, aff = S.routing(cfg)
    if N is None:
        N = mx.moe_num_blocks(cfg.T, cfg.K, cfg.E, cfg.B)
    topk_d = torch.from_numpy(topk).to(device)
    tpid, b2e = mx.moe_build_blocks(topk_d, cfg.E, cfg.B, N)
    t = S.moe_tensors(cfg, N, device)
    E, H, I = cfg.E, cfg.H, cfg.I
    gu_c, gu_s = mx.mxfp8_quantize(t["w_gate_up"].view(E * H * 2, I), 1, mx.E4M3)
    d_c, d_s = mx.mxfp8_quantize(t["w_down"].view(E * I, H), 1, mx.E4M3)
    aff_d = torch.from_numpy(aff).to(device)
    op = mx.MoeBwd(t["hidden"], aff_d, gu_c.view(E, H, 2, I), gu_s.view(E, H, 2, I // 32), d_c.view(E, I, H),
                   d_s.view(E, I, H // 32), tpid, b2e, t["dy"], cfg.B, t["ckpt"], down_proj_bias=t["b2"],
                   affinity_on=cfg.affinity_on)
    return dict(cfg=cfg, N=N, topk=topk, aff=aff, tpid=tpid, b2e=b2e, t=t, op=op,
                wq=(gu_c, gu_s, d_c, d_s))


def oracle_problem(gp, nthreads=0):
    """The oracle's view of a GPU problem: host copies of the inputs, the
    oracle's own routing blocks and weight quantisation."""
    import oracle
    from helpers import quantize_weights
    cfg = gp["cfg"]
    bits = {k: (None if v is None else S.bf16_bits(v)) for k, v in gp["t"].items()}
    tpid, b2e = oracle.build_blocks(gp["topk"], cfg.E, cfg.B, gp["N"])
    gu_c, gu_s, d_c, d_s = quantize_weights(bits["w_gate_up"], bits["w_down"])
    p = oracle.MoeProblem(T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, N=gp["N"], B=cfg.B, hidden=bits["hidden"],
                          aff=gp["aff"], wgu_codes=gu_c, wgu_scales=gu_s, wd_codes=d_c, wd_scales=d_s,
                          tpid=tpid, b2e=b2e, dy=bits["dy"], ckpt=bits["ckpt"], b2=bits["b2"],
                          affinity_on=cfg.affinity_on, has_bias=int(cfg.has_bias), nthreads=nthreads)
    return p, dict(tpid=tpid, b2e=b2e, wq=(gu_c, gu_s, d_c, d_s))


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return S.bf16_bits(t)
    return t.detach().cpu().numpy()
