"""Pins of the oracle's MX quantiser: E8M0 scale and code invariants.

The scale rule itself is a reading (the pages name MXFP8 32-element groups but
no rule): its parity with the pages is unpinned; these tests pin that the
oracle implements that reading and nothing else.
"""
import numpy as np
import pytest

import oracle

EMAX = {oracle.E4M3: 8, oracle.E5M2: 15}
MAXV = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}


def _bf16_round(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _groups(rng, n):
    out = []
    for k in range(n):
        kind = k % 6
        if kind == 0:
            v = rng.standard_normal(32)
        elif kind == 1:
            v = rng.standard_normal(32) * 10.0 ** rng.uniform(-30, 30)
        elif kind == 2:
            v = np.zeros(32); v[rng.integers(32)] = rng.standard_normal()
        elif kind == 3:
            v = rng.standard_normal(32) * 1e-39                      # bf16 subnormals
        elif kind == 4:
            v = np.zeros(32)
        else:
            v = rng.standard_normal(32) * np.where(rng.random(32) < 0.1, 1e4, 1.0)
        out.append(_bf16_round(v))
    return out


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_scale_and_code_invariants(fmt):
    rng = np.random.default_rng(1)
    for v in _groups(rng, 600):
        s, codes, deq = oracle.quantize_group(v, fmt)
        assert 0 <= s <= 254
        X = s - 127
        vals = np.array([oracle.fp8_decode(c, fmt) for c in codes])
        assert np.all(np.isfinite(vals)) and np.all(np.abs(vals) <= MAXV[fmt])
        assert np.array_equal(deq, np.ldexp(vals, X))
        assert np.array_equal(np.signbit(vals), np.signbit(v))
        amax = np.abs(v).max()
        if amax == 0:
            assert s == 0 and np.all((codes & 0x7F) == 0)
            continue
        e = int(np.floor(np.log2(amax)))
        if -127 < e - EMAX[fmt] < 127:
            y = amax * 2.0 ** -X
            assert 2.0 ** EMAX[fmt] <= y < 2.0 ** (EMAX[fmt] + 1)   # amax lands in the top binade
        else:
            assert X == -127


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_power_of_two_equivariance(fmt):
    rng = np.random.default_rng(2)
    for _ in range(200):
        v = _bf16_round(rng.standard_normal(32))
        for k in (-20, -3, 1, 7, 40):
            s0, c0, d0 = oracle.quantize_group(v, fmt)
            s1, c1, d1 = oracle.quantize_group(np.ldexp(v, k), fmt)
            assert np.array_equal(c0, c1) and s1 == s0 + k
            assert np.array_equal(np.ldexp(d0, k), d1)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_lossless_round_trip(fmt):
    """Values already on the grid of their own scale come back unchanged."""
    rng = np.random.default_rng(3)
    grid = np.array([oracle.fp8_decode(c, fmt) for c in range(256)])
    top = np.nonzero(np.isfinite(grid) & (np.abs(grid) >= 2.0 ** EMAX[fmt]))[0]
    fin = np.nonzero(np.isfinite(grid))[0]
    for _ in range(200):
        codes = rng.choice(fin, 32)
        codes[rng.integers(32)] = rng.choice(top)                  # amax in the top binade
        X = int(rng.integers(-100, 100))
        v = np.ldexp(grid[codes], X)
        s, c, d = oracle.quantize_group(v, fmt)
        assert s == X + 127
        assert np.array_equal(d, v)
        assert np.array_equal(np.array([grid[x] for x in c]), grid[codes])


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_sign_symmetry_and_axis_transpose(fmt):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    import torch
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c1, s1 = oracle.quantize(bits, 1, fmt)
    cneg, sneg = oracle.quantize(bits ^ np.uint16(0x8000), 1, fmt)
    assert np.array_equal(cneg, c1 ^ 0x80) and np.array_equal(sneg, s1)
    c0, s0 = oracle.quantize(np.ascontiguousarray(bits.T), 0, fmt)    # axis 0 of x^T
    assert np.array_equal(c0, c1.T) and np.array_equal(s0, s1.T)


def test_error_bound_half_ulp():
    """|deq - v| <= half an element ulp at the group's scale when no element saturates:
    with |v| <= 1.75 * 2^k and v[0] = 2^k, the largest y is 1.75 * 2^emax = the format max."""
    rng = np.random.default_rng(5)
    for fmt, mbits in ((oracle.E4M3, 3), (oracle.E5M2, 2)):
        for _ in range(300):
            k = int(rng.integers(-20, 20))
            v = _bf16_round(np.clip(rng.standard_normal(32) * 2.0 ** k, -1.75 * 2.0 ** k, 1.75 * 2.0 ** k))
            v[0] = 2.0 ** k
            s, c, d = oracle.quantize_group(v, fmt)
            X = s - 127
            e = np.floor(np.log2(np.maximum(np.abs(v) * 2.0 ** -X, 2.0 ** (1 - (7 if fmt == 0 else 15)))))
            half_ulp = np.ldexp(1.0, (e - mbits - 1 + X).astype(int))
            assert np.all(np.abs(d - v) <= half_ulp)
