"""Pins for the oracle's FP8 (E4M3) path against what the format and the mathematics fix:
hand-derived encodings (tests/golden), torch's float8_e4m3fn conversion (a library routine
for the same format), brute force on tiny products, and a grid-aligned layer whose codes and
outputs are exact. A wrong exponent bias, a dropped subnormal, a wrong tie rule, a missing
saturation or a wrong unit in the exact product fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_e4m3_golden_codes(golden):
    g = golden["e4m3_codes"]
    v = np.array(g["values"], dtype=np.float64)[None, :]
    q, s = O.quantize_tensor(v, O.ROT_NONE, 1, 8, O.STEP, 1.0, fmt=O.E4M3)
    assert s == 1.0
    np.testing.assert_array_equal(q[0], np.array(g["codes"], dtype=np.uint8))
    a = g["absmax_case"]
    q, s = O.quantize_tensor(np.array(a["v"])[None, :], O.ROT_NONE, 1, 8, O.ABSMAX, fmt=O.E4M3)
    assert s == np.float32(a["s"])
    np.testing.assert_array_equal(q[0], np.array(a["codes"], dtype=np.uint8))


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.decode_e4m3(codes), ref)
    assert O.decode_e4m3(np.array([0x7E], dtype=np.uint8))[0] == 448.0


def test_e4m3_quantize_matches_torch_in_range():
    """torch's float32 -> float8_e4m3fn conversion is round-to-nearest-even on the same grid;
    inside +-448 (where it does not produce NaN) the codes agree value for value, including
    every midpoint and its two fp32 neighbours."""
    pos = np.unique(np.abs(O.decode_e4m3(np.arange(0, 127, dtype=np.uint8))))
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    vals = np.concatenate([pos, mids, np.nextafter(m32, np.float32(0)).astype(np.float64),
                           np.nextafter(m32, np.float32(1e9)).astype(np.float64)])
    rng = np.random.default_rng(8)
    vals = np.concatenate([vals, rng.uniform(-448, 448, 5000), rng.normal(0, 0.01, 2000)])
    vals = vals.astype(np.float32).astype(np.float64)
    vals = np.concatenate([vals, -vals])
    q = O.quantize_e4m3(vals, 1.0)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.decode_e4m3(q), ref)


def test_e4m3_saturates_and_is_odd():
    v = np.array([448.0, 463.99, 464.0, 480.0, 1e6, 5e37])
    q = O.quantize_e4m3(np.concatenate([v, -v]), 1.0)
    np.testing.assert_array_equal(q, [0x7E] * 6 + [0xFE] * 6)
    rng = np.random.default_rng(9)
    x = rng.standard_normal(3000) * 50
    np.testing.assert_array_equal(O.decode_e4m3(O.quantize_e4m3(-x, 0.75)),
                                  -O.decode_e4m3(O.quantize_e4m3(x, 0.75)))


def test_e4m3_nearest_by_brute_force():
    """Every code is the nearest grid value times s (ties to the even code), checked with
    Fractions against the whole grid, for a non-dyadic step."""
    grid = [(c, Fraction(float(O.decode_e4m3(np.array([c], dtype=np.uint8))[0])))
            for c in range(127)]
    s = np.float32(0.3)
    rng = np.random.default_rng(10)
    R = rng.standard_normal(400) * 40
    q = O.quantize_e4m3(R, s)
    for r, c in zip(R, q):
        x = abs(Fraction(float(r)) / Fraction(float(s)))
        best = min(grid, key=lambda g: (abs(g[1] - x), g[0] & 1))
        want = best[0] if x < 448 else 126
        assert (c & 0x7F) == want and ((c >> 7) == (1 if r < 0 else 0)), (r, c, want)


def test_gemm_f8_exact_brute_force():
    rng = np.random.default_rng(11)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    A = rng.choice(codes, size=(5, 37))
    B = rng.choice(codes, size=(37, 6))
    T = O.gemm_f8(A, 37, 1, B, 6, 1, 5, 6, 37)           # units of 2^-18
    Af = [[Fraction(float(x)) for x in row] for row in O.decode_e4m3(A)]
    Bf = [[Fraction(float(x)) for x in row] for row in O.decode_e4m3(B)]
    for m in range(5):
        for n in range(6):
            exact = sum(Af[m][k] * Bf[k][n] for k in range(37))
            assert Fraction(int(T[m, n]), 2 ** 18) == exact
    # the transposed index map gives the transposed product
    Tt = O.gemm_f8(B, 1, 6, A, 1, 37, 6, 5, 37)
    np.testing.assert_array_equal(Tt, T.T)


def test_rotate_i64_overflow_raises():
    T = np.full((2, 4), 2 ** 62, dtype=np.int64)
    with pytest.raises(ValueError):
        O.rotate_i64(T, O.ROT_RIGHT, 4)


@pytest.mark.parametrize("k", [16, 32])
def test_fp8_grid_aligned_layer_exact(k):
    """X = A B_C / k with E4M3-representable A (max |A| = 448): rotate -> absmax -> quantize
    returns A with s = 1, and Y = A Bm^T / k = X W^T exactly; the HQ backward products are
    exact as well (dY on the grid with max 448)."""
    rng = np.random.default_rng(k)
    N, C, D = 2 * k, 4 * k, 3 * k
    small = O.decode_e4m3(np.arange(0x20, 0x50, dtype=np.uint8))   # values 2^-3 .. 2^3
    def draw(shape):
        v = rng.choice(small, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v[0, 0] = 448.0
        return v
    A, Bm, G = draw((N, C)), draw((D, C)), draw((N, D))
    H = np.kron(np.eye(C // k), O.hadamard(k).astype(np.float64))
    X, W = A @ H / k, Bm @ H / k
    out = O.linear(X, W, G, k, 8, O.HQ, fmt=O.E4M3)
    np.testing.assert_array_equal(O.decode_e4m3(out["qx"]), A)
    np.testing.assert_array_equal(O.decode_e4m3(out["qw"]), Bm)
    np.testing.assert_array_equal(O.decode_e4m3(out["qg"]), G)
    assert out["sx"] == out["sw"] == out["sg"] == 1.0
    np.testing.assert_array_equal(out["y"], X @ W.T)
    np.testing.assert_array_equal(out["dx"], G @ W)
    np.testing.assert_array_equal(out["dw"], G.T @ X)


@pytest.mark.parametrize("variant", [O.HQ, O.HALO0])
def test_fp8_fwd_error_bound(variant):
    """Per element, |Yhat - X W^T| <= (|e_x| . |wr| + |xr| . |e_w| + |e_x| . |e_w|) / k^e with
    |e| <= max(2^-4 |r|, 2^-10 s) elementwise: half a step of the 3-bit mantissa relative to
    the value, or half the subnormal step 2^-9 s (absmax never saturates). Nothing is
    re-typed from the oracle: the rotated values come from scipy's Hadamard matrix."""
    import scipy.linalg
    k = 32
    rng = np.random.default_rng(13)
    N, C, D = 48, 256, 64
    X = rng.standard_normal((N, C))
    X[:, [3, 77]] *= 300
    W = rng.standard_normal((D, C)) * 0.02
    out = O.linear(X, W, None, k, 8, variant, passes=("fwd",), fmt=O.E4M3)
    kk = k if variant == O.HQ else 1
    H = np.kron(np.eye(C // kk), scipy.linalg.hadamard(kk).astype(np.float64))
    xr, wr = X @ H, W @ H
    ex = np.maximum(2.0 ** -4 * np.abs(xr), 2.0 ** -10 * float(out["sx"]))
    ew = np.maximum(2.0 ** -4 * np.abs(wr), 2.0 ** -10 * float(out["sw"]))
    bound = (ex @ np.abs(wr).T + np.abs(xr) @ ew.T + ex @ ew.T) / kk
    err = np.abs(out["y"] - X @ W.T)
    assert (err <= bound * (1 + 1e-9)).all()
    # and the codes' values really are within those per-element bounds
    assert (np.abs(O.decode_e4m3(out["qx"]) * float(out["sx"]) - xr) <= ex * (1 + 1e-12)).all()
