"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds input generation only -- none of the backward's arithmetic.
Weights come out as bf16; quantising them is the caller's job (the oracle in
tests, the GPU quantiser in the benchmark).

Random numbers come from one counter-based generator, SplitMix64 (Steele, Lea
and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014):
element i of stream (seed, sid) is mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
with key = mix64(seed * 0x9E3779B97F4A7C15 + sid).  The torch version runs on
any device and gives the same bits everywhere (integer ops only); normals for
large tensors use an inverse-CDF table of 2^20 bf16 quantiles indexed by the
top 20 bits, so no transcendental function is evaluated on the device.
Routing logits are small and made on the host in float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from functools import lru_cache
from typing import Optional

import numpy as np
import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
TABLE_BITS = 20


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, sid: int) -> int:
    return _mix64_int(seed * GAMMA + sid)


# ----------------------------------------------------------------------------- numpy (host)
def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(MIX1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def bits_np(n: int, seed: int, sid: int, start: int = 0) -> np.ndarray:
    key = np.uint64(stream_key(seed, sid))
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64_np(key + i * np.uint64(GAMMA))


def uniform_np(n: int, seed: int, sid: int) -> np.ndarray:
    """Uniforms in (0,1): (top 53 bits + 0.5) * 2^-53."""
    return ((bits_np(n, seed, sid) >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def normal_np(n: int, seed: int, sid: int) -> np.ndarray:
    """Box-Muller N(0,1) in float64 from two uniform streams (host only)."""
    u1 = uniform_np(n, seed, sid)
    u2 = uniform_np(n, seed, sid + 0x5151)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def gumbel_np(n: int, seed: int, sid: int) -> np.ndarray:
    return -np.log(-np.log(uniform_np(n, seed, sid)))


# ----------------------------------------------------------------------------- torch (any device)
def _s64(c: int) -> int:
    return c - (1 << 64) if c >= (1 << 63) else c


def _srl(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _srl(z, 30)
    z = z * _s64(MIX1)
    z = z ^ _srl(z, 27)
    z = z * _s64(MIX2)
    return z ^ _srl(z, 31)


def bits_t(n: int, seed: int, sid: int, device, start: int = 0) -> torch.Tensor:
    key = _s64(stream_key(seed, sid))
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64_t(i * _s64(GAMMA) + key)


@lru_cache(maxsize=32)
def _normal_table_host(sigma: float) -> torch.Tensor:
    from scipy.special import ndtri
    k = np.arange(1 << TABLE_BITS, dtype=np.float64)
    q = ndtri((k + 0.5) / float(1 << TABLE_BITS)) * sigma
    return torch.from_numpy(q).to(torch.bfloat16)


_dev_tables: dict = {}


def _normal_table(sigma: float, device) -> torch.Tensor:
    key = (float(sigma), str(device))
    if key not in _dev_tables:
        _dev_tables[key] = _normal_table_host(float(sigma)).to(device)
    return _dev_tables[key]


def normal_bf16(shape, sigma: float, seed: int, sid: int, device="cpu",
                chunk: int = 1 << 26) -> torch.Tensor:
    """bf16 tensor of N(0, sigma^2) samples (inverse-CDF table, 2^20 levels)."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    tab = _normal_table(sigma, device)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        idx = _srl(bits_t(m, seed, sid, device, start=s), 64 - TABLE_BITS)
        out[s:s + m] = tab[idx]
    return out.view(*shape)


def int_bits_t(n: int, seed: int, sid: int, device="cpu") -> torch.Tensor:
    """Raw 64-bit stream as int64 (for generator self-checks)."""
    return bits_t(n, seed, sid, device)


# ----------------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class MoeConfig:
    """One MoE backward workload: shapes, routing law and layer options."""
    name: str
    T: int
    H: int
    I: int
    E: int
    K: int
    B: int
    routing: str              # "normal" | "zipf" | "hotcold"
    affinity_on: int = 0      # 0 = affinity on H (output), 1 = on I (intermediate)
    has_bias: bool = False
    zipf_s: float = 1.1
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.T * self.K

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs of the backward: 12*H*I per routed pair (2HI + 4HI + 4HI + 2HI)."""
        return 12 * self.pairs * self.H * self.I


@dataclass(frozen=True)
class DenseConfig:
    name: str
    M: int
    N: int
    K: int
    seed: int = 0

    @property
    def flops(self) -> int:
        return 4 * self.M * self.N * self.K


TINY = MoeConfig("tiny_T256_H128_I256_E4_top2_B128", 256, 128, 256, 4, 2, 128, "normal")
DENSE = DenseConfig("dense_M4096_N4096_K4096", 4096, 4096, 4096)
MEDIUM = MoeConfig("medium_T8192_H2048_I1408_E16_top4zipf_B512", 8192, 2048, 1408, 16, 4, 512, "zipf")
LARGE = MoeConfig("large_T16384_H4096_I14336_E8_top2_B1024_onI", 16384, 4096, 14336, 8, 2, 1024,
                  "normal", affinity_on=1)
FINE = MoeConfig("fine_T32768_H1536_I256_E128_top8hot_B128_bias", 32768, 1536, 256, 128, 8, 128,
                 "hotcold", has_bias=True)
MOE_CONFIGS = {"tiny": TINY, "medium": MEDIUM, "large": LARGE, "fine": FINE}

# stream ids, one per tensor
SID_LOGIT, SID_GUMBEL, SID_X, SID_DY, SID_WGU, SID_WD, SID_CKPT, SID_B2 = 1, 2, 3, 4, 5, 6, 7, 8
SID_DENSE_X, SID_DENSE_W, SID_DENSE_DY = 11, 12, 13

HOT_LOAD = 3.0   # fine-grained law: ~20% of experts (26 of 128) take 3x the mean load and
                 # 1 in 16 (8 of 128) get no tokens; the rest share what is left equally


def hot_cold_counts(E: int):
    return max(1, round(E * 26 / 128)), max(1, round(E / 16))


def router_logits(cfg: MoeConfig) -> np.ndarray:
    """[T,E] float64 logits; -inf marks experts that can never be chosen."""
    T, E = cfg.T, cfg.E
    if cfg.routing == "normal":
        return normal_np(T * E, cfg.seed, SID_LOGIT).reshape(T, E)
    g = gumbel_np(T * E, cfg.seed, SID_GUMBEL).reshape(T, E)
    if cfg.routing == "zipf":
        w = (np.arange(E, dtype=np.float64) + 1.0) ** (-cfg.zipf_s)
    elif cfg.routing == "hotcold":
        hot, empty = hot_cold_counts(E)
        w = np.zeros(E)
        w[:hot] = HOT_LOAD
        w[hot:E - empty] = (E - HOT_LOAD * hot) / (E - hot - empty)
    else:
        raise ValueError(cfg.routing)
    with np.errstate(divide="ignore"):
        return np.log(w / w.sum())[None, :] + g


def routing(cfg: MoeConfig):
    """(topk_ids [T,K] int32, affinities [T*E] float32).

    Top-k by logit (ties: lower expert id first); affinity = softmax over all E
    logits, kept only at the chosen experts ("masked")."""
    lg = router_logits(cfg)
    order = np.argsort(-lg, axis=1, kind="stable")
    topk = np.ascontiguousarray(order[:, :cfg.K].astype(np.int32))
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    p /= p.sum(axis=1, keepdims=True)
    aff = np.zeros_like(p)
    rows = np.arange(cfg.T)[:, None]
    aff[rows, topk] = p[rows, topk]
    return topk, aff.astype(np.float32).reshape(-1)


def moe_tensors(cfg: MoeConfig, N: int, device="cpu"):
    """bf16 tensors of one MoE workload.  N (blocks) sizes the checkpoint.

    hidden, dy ~ N(0,1) [T,H]; w_gate_up ~ N(0,0.02) [E,H,2,I]; w_down ~ N(0,0.02)
    [E,I,H]; the gate/up checkpoint [N,2,I,B] is i.i.d. N(0, 0.02*sqrt(H)), the
    spread of x.W for these x and W (padding slots hold samples too, which the
    backward must ignore); b2 ~ N(0,0.02) [E,H] when the layer has a bias."""
    s = cfg.seed
    out = dict(
        hidden=normal_bf16((cfg.T, cfg.H), 1.0, s, SID_X, device),
        dy=normal_bf16((cfg.T, cfg.H), 1.0, s, SID_DY, device),
        w_gate_up=normal_bf16((cfg.E, cfg.H, 2, cfg.I), 0.02, s, SID_WGU, device),
        w_down=normal_bf16((cfg.E, cfg.I, cfg.H), 0.02, s, SID_WD, device),
        ckpt=normal_bf16((N, 2, cfg.I, cfg.B), 0.02 * math.sqrt(cfg.H), s, SID_CKPT, device),
    )
    out["b2"] = normal_bf16((cfg.E, cfg.H), 0.02, s, SID_B2, device) if cfg.has_bias else None
    return out


def dense_tensors(cfg: DenseConfig, device="cpu"):
    """X [M,K] ~ N(0,1), W [N,K] ~ N(0,0.02), dY [M,N] ~ N(0,1), all bf16."""
    s = cfg.seed
    return dict(
        x=normal_bf16((cfg.M, cfg.K), 1.0, s, SID_DENSE_X, device),
        w=normal_bf16((cfg.N, cfg.K), 0.02, s, SID_DENSE_W, device),
        dy=normal_bf16((cfg.M, cfg.N), 1.0, s, SID_DENSE_DY, device),
    )


def scaled(cfg: MoeConfig, **kw) -> MoeConfig:
    """Same workload law at other sizes (for parity cases the oracle finishes quickly)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    if "name" not in kw:
        d["name"] = f"{cfg.name.split('_')[0]}_T{d['T']}_H{d['H']}_I{d['I']}_E{d['E']}_K{d['K']}_B{d['B']}"
    return MoeConfig(**d)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(device)
