"""Pins for the oracle's batched HQ-MM (INT4 page §A.1): it is built only from the pinned
single-layer steps, so these check the composition itself - one batch is the layer, batches
with a shared step are independent layers, and the shared absmax scale is the largest of the
batches' own scales (a misplaced slice, a per-batch scale or a rotation block that crosses a
batch fails one of them)."""
import numpy as np
import pytest

import oracle as O


def _inputs(rng, nb, N, C, D):
    X = rng.standard_normal((nb, N, C))
    X[:, :, 3] *= 30
    W = rng.standard_normal((nb, D, C))
    G = rng.standard_normal((nb, N, D)) * 1e-3
    return X, W, G


@pytest.mark.parametrize("variant", [O.HALO2, O.HQ, O.HALO0])
def test_one_batch_is_the_layer(variant):
    rng = np.random.default_rng(1)
    X, W, G = _inputs(rng, 1, 32, 64, 48)
    a = O.linear_batched(X, W, G, 16, 8, variant)
    b = O.linear(X[0], W[0], G[0], 16, 8, variant)
    for key in ("y", "dx", "dw"):
        np.testing.assert_array_equal(a[key][0], b[key])
    for key in ("qx", "qw", "qg", "qxt"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("fmt", [O.INT, O.E4M3])
def test_shared_step_batches_are_independent_layers(fmt):
    """With given steps the tensor-wise scale is the same for every batch, so batch b of the
    batched product is the layer of batch b alone (HALO-2: token blocks stay in a batch)."""
    rng = np.random.default_rng(2)
    nb, N, C, D, k = 3, 32, 64, 48, 16
    X, W, G = _inputs(rng, nb, N, C, D)
    steps = {"x": 0.9, "xt": 3.0, "w": 0.2, "g": 4e-5}
    bits = 8
    mode = O.STEP
    a = O.linear_batched(X, W, G, k, bits, O.HALO2, mode, steps, fmt=fmt)
    for bi in range(nb):
        b = O.linear(X[bi], W[bi], G[bi], k, bits, O.HALO2, mode, steps, fmt=fmt)
        for key in ("y", "dx", "dw"):
            np.testing.assert_array_equal(a[key][bi], b[key])


def test_shared_absmax_scale_is_the_largest_batch_scale():
    rng = np.random.default_rng(3)
    nb, N, C, D, k = 4, 32, 64, 48, 16
    X, W, G = _inputs(rng, nb, N, C, D)
    X[2] *= 5                                  # one batch dominates
    a = O.linear_batched(X, W, G, k, 8, O.HALO2)
    per = [O.linear(X[b], W[b], G[b], k, 8, O.HALO2) for b in range(nb)]
    for key in ("sx", "sxt", "sw", "sg"):
        assert a[key] == max(p[key] for p in per), key
    # the dominating batch's codes are its own layer's codes (same scale there)
    np.testing.assert_array_equal(a["qx"][2 * N:3 * N], per[2]["qx"])
