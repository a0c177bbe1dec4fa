"""Pins for the oracle's LSS-MM weight gradient (INT4 page §4.2, §A.2, §A.3, §A.6, §B.2):
hand-derived probabilities (tests/golden), the probability rule's invariants, unbiasedness of
the row-sampled estimator by enumerating every mask on a small case, the bit split's identity
with a single rounding, and the no-sampling limit against the exact product."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def test_probabilities_golden():
    with open(GOLDEN) as f:
        g = json.load(f)["lss_probabilities"]
    for c in g["cases"]:
        p = O.lss_probabilities(c["scores"], c["budget"])
        want = c["p"] if "p" in c else [v / c["p_den"] for v in c["p_num"]]
        np.testing.assert_allclose(p, want, rtol=1e-15, atol=0)


@pytest.mark.parametrize("seed", range(5))
def test_probabilities_invariants(seed):
    rng = np.random.default_rng(seed)
    n = 200
    l = rng.lognormal(0, 2.5, n) * (rng.random(n) < 0.8)
    budget = rng.uniform(5, 150)
    p = O.lss_probabilities(l, budget)
    assert (p >= 0).all() and (p <= 1).all()
    assert (p[l == 0] == 0).all()
    if budget <= np.count_nonzero(l):
        assert abs(p.sum() - budget) <= 1e-9 * budget
    free = (p > 0) & (p < 1)
    ratio = p[free] / l[free]                       # proportional to the score when unclamped
    assert np.allclose(ratio, ratio[0], rtol=1e-12)
    if free.any():                                   # clamped entries have the larger scores
        assert l[p == 1].min(initial=np.inf) >= l[free].max() * (1 - 1e-12)


def test_row_sampling_is_unbiased_by_enumeration():
    """E over the Bernoulli masks of sum_i m_i / p_i g_i^T x_i equals sum_i g_i^T x_i exactly
    (Fractions, every one of the 2^6 masks weighted by its probability)."""
    rng = np.random.default_rng(7)
    N, D, C = 6, 3, 4
    G = rng.integers(-5, 6, size=(N, D))
    X = rng.integers(-5, 6, size=(N, C))
    l = np.sqrt((G * G).sum(1) * (X * X).sum(1))
    p = [Fraction(v).limit_denominator(1 << 40) for v in O.lss_probabilities(l, 3)]
    exact = [[Fraction(int(sum(G[i, d] * X[i, c] for i in range(N)))) for c in range(C)]
             for d in range(D)]
    expect = [[Fraction(0)] * C for _ in range(D)]
    for mask in itertools.product([0, 1], repeat=N):
        prob = Fraction(1)
        for i in range(N):
            prob *= p[i] if mask[i] else 1 - p[i]
        if prob == 0:
            continue
        for d in range(D):
            for c in range(C):
                expect[d][c] += prob * sum(Fraction(int(G[i, d] * X[i, c])) / p[i]
                                           for i in range(N) if mask[i])
    assert expect == exact


def test_bit_split_is_one_rounding_on_the_fine_grid():
    """hi = Q_7(v / s_hi), lo = Q_7((v - s_hi hi) / s_lo) with s_lo = s_hi / 14 give
    14 hi + lo = RNE(v / s_lo): the residual of a nearest-rounding hi never leaves [-7, 7] fine
    steps, so the split is an INT8-range code split into two INT4 codes."""
    rng = np.random.default_rng(8)
    G = rng.standard_normal((40, 24)) * np.where(rng.random((40, 1)) < 0.3, 20, 0.5)
    X = rng.standard_normal((40, 32))
    qx, sx = O.quantize_tensor(X, O.ROT_RIGHT, 16, 4)
    u = np.zeros(40, dtype=np.float32)                  # keep every token with p > 0
    out = O.lss_weight_gradient(G, qx, sx, 16, 40, u)
    assert np.abs(out["hi"]).max() <= 7 and np.abs(out["lo"]).max() <= 7
    Gw = G[out["keep"]] / out["p"][out["keep"]][:, None]
    single = O.quantize(Gw, out["s_lo"], 127).astype(np.int64)
    np.testing.assert_array_equal(14 * out["hi"].astype(np.int64) + out["lo"], single)
    assert out["s_lo"] == np.float32(float(out["s_hi"]) / 14)


def test_no_sampling_limit_matches_the_product():
    """With a budget covering every token all nonzero rows are kept with p = 1; the result is
    then G^T X with the gradient on the fine grid and X on its INT4 codes: within the
    per-element quantization bound of the exact product."""
    rng = np.random.default_rng(9)
    N, C, D, k = 48, 64, 20, 16
    G = rng.standard_normal((N, D))
    G[5] = 0.0                                           # a zero row is never kept
    X = rng.standard_normal((N, C))
    qx, sx = O.quantize_tensor(X, O.ROT_RIGHT, k, 4)
    out = O.lss_weight_gradient(G, qx, sx, k, N, np.zeros(N, dtype=np.float32))
    assert 5 not in out["keep"] and len(out["keep"]) == N - 1
    H = np.kron(np.eye(C // k), scipy.linalg.hadamard(k).astype(np.float64))
    Xhat = (qx.astype(np.float64) * float(sx)) @ H / k           # X as its codes stand for it
    ref = G.T @ Xhat
    eg = float(out["s_lo"]) / 2                                  # gradient error per element
    bound = eg * np.abs(Xhat).sum(0)[None, :] * np.ones((D, 1))
    assert (np.abs(out["dw"] - ref) <= bound * (1 + 1e-9) + 1e-12).all()
