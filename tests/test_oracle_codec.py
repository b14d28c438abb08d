"""Pins of the oracle's element codec and bf16 rounding.

Against: torch's float8_e4m3fn / float8_e5m2 dtypes (a library's decode and its
round-to-nearest-even cast), a brute-force nearest-grid search, and the
hand-worked groups in tests/golden/mx_groups.json.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

FMTS = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
MAXV = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_matches_torch_float8(fmt):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(FMTS[fmt]).to(torch.float64).numpy()
    mine = np.array([oracle.fp8_decode(c, fmt) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = oracle.bf16_to_float(bits).astype(np.float64)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_matches_torch_cast_in_range(fmt):
    """In range (|y| <= max) the oracle's RNE equals torch's cast."""
    v = _all_finite_bf16()
    ys = []
    for s in range(-40, 41, 3):
        y = np.ldexp(v, s)
        ys.append(y[(np.abs(y) <= MAXV[fmt]) & (np.abs(y) >= 2.0 ** -126)])
    y = np.concatenate(ys + [np.array([0.0, -0.0])])
    assert np.array_equal(y.astype(np.float32).astype(np.float64), y)  # exact in fp32
    ref = torch.from_numpy(y.astype(np.float32)).to(FMTS[fmt]).view(torch.uint8).numpy()
    mine = oracle.fp8_encode_array(y, fmt)
    bad = np.nonzero(ref != mine)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. y={y[bad[:5]]} ref={ref[bad[:5]]} mine={mine[bad[:5]]}"


def _nearest_code_bruteforce(y, fmt):
    """Nearest finite grid value by search; ties -> even code; beyond max -> max."""
    grid_codes = np.arange(0x80)
    grid = np.array([oracle.fp8_decode(c, fmt) for c in grid_codes])
    fin = np.isfinite(grid)
    grid, grid_codes = grid[fin], grid_codes[fin]          # ascending in value and code
    a = np.abs(y)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, grid.size - 1)
    lo = np.clip(hi - 1, 0, grid.size - 1)
    dlo, dhi = np.abs(a - grid[lo]), np.abs(grid[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (grid_codes[hi] % 2 == 0))
    code = np.where(pick_hi, grid_codes[hi], grid_codes[lo])
    code = np.where(a >= grid[-1], grid_codes[-1], code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_bruteforce_all_bf16_and_ties(fmt):
    v = _all_finite_bf16()
    grid = np.array([oracle.fp8_decode(c, fmt) for c in range(0x80)])
    grid = grid[np.isfinite(grid)]
    mids = (grid[:-1] + grid[1:]) / 2                       # exact ties
    extra = np.concatenate([mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                            grid * 1.5, grid[-1] * np.array([1.01, 1.1, 2.0, 1e6])])
    ys = [np.ldexp(v, s) for s in range(-24, 25, 4)] + [extra]
    y = np.concatenate(ys)
    ref = _nearest_code_bruteforce(y, fmt)
    mine = oracle.fp8_encode_array(y, fmt)
    bad = np.nonzero(ref != mine)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. y={y[bad[:5]]}"


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),      # bf16 subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 3.0e38, -3.0e38], np.float32),
    ])
    # exact ties: bf16 value + half its quantum
    b = torch.from_numpy(x[:1000]).to(torch.bfloat16).to(torch.float32).numpy()
    tie = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, tie])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.double_to_bf16(float(t)) for t in x], np.uint16)
    assert np.array_equal(ref, mine)


def test_golden_groups():
    path = os.path.join(os.path.dirname(__file__), "golden", "mx_groups.json")
    g = json.load(open(path))
    for grp in g["groups"]:
        vals = np.zeros(32)
        vals[:len(grp["values"])] = [float(s) for s in grp["values"]]
        scale, codes, _ = oracle.quantize_group(vals, grp["fmt"])
        want = np.zeros(32, np.uint8)
        want[:len(grp["codes"])] = [int(c, 16) for c in grp["codes"]]
        assert scale == grp["scale"], grp["why"]
        assert np.array_equal(codes, want), (grp["why"], codes[:len(grp["codes"])])
