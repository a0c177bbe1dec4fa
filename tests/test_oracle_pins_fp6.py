"""Pins for the oracle's FP6 (E2M3, E3M2) codes against what the formats and the mathematics
fix: hand-listed grids and hand-derived encodings (tests/golden), torch's float8_e4m3fn decode
of the stored bytes and its conversion on the range where E2M3 shares E4M3's 3-bit mantissa (a
library routine for a related format), brute force over the hand-listed grids for the nearest
value and its tie, the correctly rounded scale as an exact fraction, and grid-aligned layers
whose codes and outputs are exact. A wrong bias, a dropped subnormal, a wrong tie rule, a
missing saturation or a wrong E4M3 embedding fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
FMTS = {"e2m3": O.E2M3, "e3m2": O.E3M2}


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)["fp6_codes"]


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_golden_codes(golden, name):
    fmt = FMTS[name]
    g = golden[name]
    v = np.array(g["values"], dtype=np.float64)[None, :]
    q, s = O.quantize_tensor(v, O.ROT_NONE, 1, 6, O.STEP, 1.0, fmt=fmt)
    assert s == 1.0
    np.testing.assert_array_equal(q[0], np.array(g["codes"], dtype=np.uint8))
    a = golden[name + "_absmax"]
    q, s = O.quantize_tensor(np.array(a["v"])[None, :], O.ROT_NONE, 1, 6, O.ABSMAX, fmt=fmt)
    assert s == np.float32(a["s"])
    np.testing.assert_array_equal(q[0], np.array(a["codes"], dtype=np.uint8))


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_grid_is_the_hand_listed_one(golden, name):
    """The values the quantizer can produce are exactly the hand-listed grid, each grid value
    maps to itself, and the grid bound is its largest value."""
    fmt = FMTS[name]
    grid = np.array(golden[name + "_grid"], dtype=np.float64)
    assert O.fp6_max(fmt) == grid[-1] == O.qmax(6, fmt)
    np.testing.assert_array_equal(O.decode_e4m3(O.quantize_fp6(grid, 1.0, fmt)), grid)
    np.testing.assert_array_equal(O.decode_e4m3(O.quantize_fp6(-grid[1:], 1.0, fmt)), -grid[1:])
    sweep = np.linspace(-2 * grid[-1], 2 * grid[-1], 40001)
    got = np.unique(np.abs(O.decode_e4m3(O.quantize_fp6(sweep, 1.0, fmt))))
    np.testing.assert_array_equal(got, grid)


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_bytes_decode_with_torch(golden, name):
    """The stored bytes are E4M3 encodings: torch's float8_e4m3fn decodes them to the grid."""
    fmt = FMTS[name]
    grid = np.array(golden[name + "_grid"], dtype=np.float64)
    vals = np.concatenate([grid, -grid[1:]])
    q = O.quantize_fp6(vals, 1.0, fmt)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ref, vals)


def test_e2m3_normal_range_is_e4m3_rounding():
    """Between 1 and 7.5 E2M3 and E4M3 have the same 3-bit mantissa, so rounding to E2M3 there
    is torch's float32 -> float8_e4m3fn conversion (round to nearest even), midpoints included."""
    grid = np.unique(np.abs(O.decode_e4m3(O.quantize_fp6(np.linspace(1, 7.5, 200), 1.0, O.E2M3))))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(61)
    vals = np.concatenate([grid, mids, rng.uniform(1.0, 7.5, 5000)])
    vals = vals.astype(np.float32).astype(np.float64)
    vals = np.concatenate([vals, -vals])
    got = O.decode_e4m3(O.quantize_fp6(vals, 1.0, O.E2M3))
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_nearest_by_brute_force(golden, name):
    """Every code is the nearest hand-listed grid value times s, a tie going to the even
    position in the grid (the even mantissa), saturating, with a non-dyadic step; checked with
    Fractions."""
    fmt = FMTS[name]
    grid = [(i, Fraction(x)) for i, x in enumerate(golden[name + "_grid"])]
    top = grid[-1][1]
    s = np.float32(0.3)
    rng = np.random.default_rng(62 + fmt)
    R = rng.standard_normal(600) * float(top) * 0.2
    R = np.concatenate([R, [float(top) * 0.3 * 2, -float(top)]])   # two beyond the grid
    # exact midpoints times s are ties: they must go to the even neighbour
    mids = [float((grid[i][1] + grid[i + 1][1]) / 2 * Fraction(float(s))) for i in range(len(grid) - 1)]
    mids = [m for m in mids if Fraction(m) / Fraction(float(s)) in
            {(grid[i][1] + grid[i + 1][1]) / 2 for i in range(len(grid) - 1)}]
    R = np.concatenate([R, mids, [-m for m in mids]])
    q = O.quantize_fp6(R, s, fmt)
    got = O.decode_e4m3(q)
    for r, c, v in zip(R, q, got):
        x = abs(Fraction(float(r)) / Fraction(float(s)))
        best = top if x >= top else min(grid, key=lambda g: (abs(g[1] - x), g[0] & 1))[1]
        assert Fraction(abs(float(v))) == best, (r, v, best)
        assert (c >> 7) == (1 if r < 0 else 0)


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_fp6_scale_is_correctly_rounded(name):
    """s = fp32(max|R| / largest value), the exact quotient rounded once to nearest even."""
    fmt = FMTS[name]
    top = Fraction(O.fp6_max(fmt))
    rng = np.random.default_rng(63 + fmt)
    for a in np.concatenate([rng.uniform(1e-3, 1e3, 300), [1.0, 3.0, 7.5, 28.0, 0.1]]):
        s = O.absmax_scale(np.array([a, -a / 3]), float(top))
        exact = Fraction(float(a)) / top
        lo, hi = np.nextafter(s, np.float32(0)), np.nextafter(s, np.float32(np.inf))
        assert abs(Fraction(float(s)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(s)) - exact) <= abs(Fraction(float(hi)) - exact)


@pytest.mark.parametrize("name,k", [("e2m3", 16), ("e3m2", 32)])
def test_fp6_grid_aligned_layer_exact(golden, name, k):
    """X = A B_C / k with A on the FP6 grid (one entry at the largest value): rotate -> absmax
    -> quantize returns A with s = 1, and Y = X W^T, dX = dY W and dW = dY^T X come out exact
    under HQ (the FP8 product of the stored bytes is exact)."""
    fmt = FMTS[name]
    rng = np.random.default_rng(64 + k)
    grid = np.array(golden[name + "_grid"][1:], dtype=np.float64)
    N, C, D = 2 * k, 4 * k, 3 * k

    def draw(shape):
        v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v[0, 0] = grid[-1]
        return v
    A, Bm, G = draw((N, C)), draw((D, C)), draw((N, D))
    H = np.kron(np.eye(C // k), O.hadamard(k).astype(np.float64))
    X, W = A @ H / k, Bm @ H / k
    out = O.linear(X, W, G, k, 6, O.HQ, fmt=fmt)
    np.testing.assert_array_equal(O.decode_e4m3(out["qx"]), A)
    np.testing.assert_array_equal(O.decode_e4m3(out["qw"]), Bm)
    np.testing.assert_array_equal(O.decode_e4m3(out["qg"]), G)
    assert out["sx"] == out["sw"] == out["sg"] == 1.0
    np.testing.assert_array_equal(out["y"], X @ W.T)
    np.testing.assert_array_equal(out["dx"], G @ W)
    np.testing.assert_array_equal(out["dw"], G.T @ X)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E2M3, O.E3M2])
def test_zero_codes_keep_the_sign_bit(fmt):
    """A value that rounds to zero keeps its IEEE sign: -0.0 and tiny negatives give 0x80,
    +0.0 and tiny positives 0x00."""
    vals = np.array([0.0, -0.0, 1e-30, -1e-30])
    q = O.quantize_e4m3(vals, 1.0) if fmt == O.E4M3 else O.quantize_fp6(vals, 1.0, fmt)
    np.testing.assert_array_equal(q, [0x00, 0x80, 0x00, 0x80])


def test_fp6_formats_are_6_bits():
    with pytest.raises(ValueError):
        O.qmax(8, O.E2M3)
    with pytest.raises(ValueError):
        O.qmax(4, O.E3M2)
    with pytest.raises(ValueError):
        O.quantize_fp6(np.zeros(3), 1.0, O.E4M3)
