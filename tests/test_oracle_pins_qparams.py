"""Pins for the oracle's quantizer-parameter statistics (INT4 page §3.1, §A.3-§A.5): a
hand-derived example (tests/golden), torch autograd of a learned-step quantizer written with
straight-through rounding (an independent route to the step gradient), grid-aligned inputs
with zero quantization error, and the selection rule on a case whose answer is forced."""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)["quantizer_parameters_k2"]


def test_stats_golden(golden):
    V = np.array(golden["v"], dtype=np.float64)
    G = np.array(golden["g"], dtype=np.float64)
    st = O.rotated_stats(V, G, O.ROT_RIGHT, golden["k"], golden["bits"], golden["step"])
    assert st["abs_sum"] == golden["abs_sum"]
    assert st["qerr"] == golden["qerr"]
    assert st["lsq"] == golden["lsq"]
    s = O.cold_start_step(V, O.ROT_RIGHT, golden["k"], golden["bits"])
    assert abs(float(s) - golden["cold_start_step"]) <= float(np.spacing(np.float32(s)))


@pytest.mark.parametrize("bits", [4, 8])
def test_lsq_gradient_matches_torch_autograd(bits):
    """A learned-step quantizer in torch: x = clamp(v / s, -Qp, Qp), straight-through RNE
    rounding (torch.round rounds halves to even), v_hat = s * x_q; the loss sum(g * v_hat)
    differentiated by autograd with respect to s equals the oracle's lsq statistic."""
    qp = O.qmax(bits)
    rng = np.random.default_rng(bits)
    k = 16
    V = rng.standard_normal((12, 64)) * np.where(rng.random((12, 64)) < 0.05, 20, 1)
    G = rng.standard_normal((12, 64))
    H = np.kron(np.eye(64 // k), scipy.linalg.hadamard(k).astype(np.float64))
    R = V @ H
    step = np.float32(np.abs(R).mean() * 2 / np.sqrt(qp))
    s = torch.tensor(float(step), dtype=torch.float64, requires_grad=True)
    v = torch.from_numpy(R)
    x = torch.clamp(v / s, -qp, qp)
    xq = x + (torch.round(x) - x).detach()
    loss = (torch.from_numpy(G @ H / k) * (xq * s)).sum()
    loss.backward()
    st = O.rotated_stats(V, G, O.ROT_RIGHT, k, bits, step)
    assert abs(st["lsq"] - float(s.grad)) <= 1e-9 * max(1.0, abs(float(s.grad)))


@pytest.mark.parametrize("k", [4, 16])
def test_qerr_zero_on_grid_and_bounded(k):
    """Rotated values on the step grid have no quantization error; otherwise each entry's
    error is at most s/2 (no clipping under absmax), so qerr <= n s^2 / 4."""
    rng = np.random.default_rng(k)
    A = rng.integers(-127, 128, size=(8, 4 * k)).astype(np.float64)
    H = np.kron(np.eye(4), scipy.linalg.hadamard(k).astype(np.float64))
    V = A @ H / k
    assert O.rotated_stats(V, None, O.ROT_RIGHT, k, 8, 1.0)["qerr"] == 0.0
    V = rng.standard_normal((8, 4 * k))
    R = V @ H
    s = O.absmax_scale(R, 127)
    st = O.rotated_stats(V, None, O.ROT_RIGHT, k, 8, s)
    assert 0 < st["qerr"] <= R.size * float(s) ** 2 / 4


def test_choose_k_forced_by_a_grid_aligned_activation():
    """X B_8 lies on its absmax grid (X = A B_8 / 8 with integer A, max 127), so k = 8 gives
    zero activation error and a zero product: the rule must pick 8 among the candidates."""
    rng = np.random.default_rng(4)
    A = rng.integers(-127, 128, size=(16, 64)).astype(np.float64)
    A[0, 0] = 127
    H8 = np.kron(np.eye(8), scipy.linalg.hadamard(8).astype(np.float64))
    X = A @ H8 / 8
    W = rng.standard_normal((24, 64))
    best, errs = O.choose_hadamard_k(X, W, [1, 2, 4, 8, 16, 32], 8)
    assert best == 8 and errs[8][0] == 0.0
    assert all(errs[k][0] > 0 for k in (1, 2, 4, 16, 32))


def test_choose_k_prefers_rotation_with_outliers():
    """Direction check (INT4 page §3.2-§3.3): with a few outlier channels, some rotated size
    beats no rotation (k = 1)."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((64, 256))
    X[:, [7, 100]] *= 80
    W = rng.standard_normal((48, 256)) * 0.02
    best, errs = O.choose_hadamard_k(X, W, [1, 16, 64, 256], 4)
    assert best != 1
    assert errs[best][0] * errs[best][1] < errs[1][0] * errs[1][1]
