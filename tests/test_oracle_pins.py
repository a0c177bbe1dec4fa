"""Pins for the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own formulas: they use hand-derived worked
examples (tests/golden), textbook constructions (Sylvester recursion, scipy's Hadamard),
closed forms, invariants, exact product identities on tiny integer inputs, brute force, and
a derived per-element error bound. A dropped term, a wrong sign or index, a transposed
operand, a wrong exponent of k or a wrong rotation side in the oracle fails at least one.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def blockdiag_h(n, k):
    """Dense block-diagonal Hadamard from scipy's (Sylvester, natural order) H_k."""
    return np.kron(np.eye(n // k), scipy.linalg.hadamard(k)).astype(np.float64)


# ------------------------------------------------------------------------ H_k
@pytest.mark.parametrize("k", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_sylvester_recursion(k):
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < k:
        H = np.block([[H, H], [H, -H]])
    np.testing.assert_array_equal(O.hadamard(k).astype(np.int64), H)


@pytest.mark.parametrize("k", [2, 4, 16, 256])
def test_hadamard_orthogonality_symmetry(k):
    H = O.hadamard(k).astype(np.int64)
    np.testing.assert_array_equal(H @ H.T, k * np.eye(k, dtype=np.int64))   # H H^T = k I
    np.testing.assert_array_equal(H, H.T)
    assert (H[0] == 1).all() and (H[:, 0] == 1).all()
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(k))


def test_hadamard_golden(golden):
    for k, mat in golden["hadamard"].items():
        if k.startswith("_"):
            continue
        np.testing.assert_array_equal(O.hadamard(int(k)), np.array(mat))


@pytest.mark.parametrize("k", [0, 3, 12, 512, -4])
def test_hadamard_rejects_bad_k(k):
    with pytest.raises(ValueError):
        O.hadamard(k)


# ------------------------------------------------------------------ decoding
def test_decode_matches_numpy():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(4096) * np.exp(rng.uniform(-20, 10, 4096))).astype(np.float32)
    h = v.astype(np.float16)
    np.testing.assert_array_equal(O.decode(h.view(np.uint16), O.F16), h.astype(np.float64))
    b = (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # exact bf16 values
    bits = (b.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    np.testing.assert_array_equal(O.decode(bits, O.BF16), b.astype(np.float64))
    np.testing.assert_array_equal(O.decode(v, O.F32), v.astype(np.float64))


def test_round_to_matches_numpy_and_torch():
    import torch
    rng = np.random.default_rng(1)
    v32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 9, 20000))).astype(np.float32)
    v = v32.astype(np.float64)
    np.testing.assert_array_equal(O.round_to(v, O.F16), v.astype(np.float16).view(np.uint16))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.round_to(v, O.BF16), ref)
    np.testing.assert_array_equal(O.round_to(v, O.F32), v32)
    # exact ties: 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7 -> even (1)
    assert O.round_to(np.array([1 + 2.0 ** -8]), O.BF16)[0] == 0x3F80
    assert O.round_to(np.array([1 + 3 * 2.0 ** -8]), O.BF16)[0] == 0x3F82


# ----------------------------------------------------------------- rotations
@pytest.mark.parametrize("k", [1, 2, 4, 8, 32])
def test_rotation_matches_blockdiag_matmul(k):
    rng = np.random.default_rng(k)
    V = rng.standard_normal((2 * k, 4 * k))
    np.testing.assert_allclose(O.rotate(V, O.ROT_RIGHT, k), V @ blockdiag_h(4 * k, k),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.rotate(V, O.ROT_LEFT, k), blockdiag_h(2 * k, k) @ V,
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.rotate(V, O.ROT_BOTH, k),
                               blockdiag_h(2 * k, k) @ V @ blockdiag_h(4 * k, k),
                               rtol=0, atol=1e-11)


@pytest.mark.parametrize("k", [2, 16, 256])
def test_rotation_round_trip_exact(k):
    rng = np.random.default_rng(7)
    V = rng.integers(-50, 50, size=(k, 2 * k)).astype(np.float64)
    for rot in (O.ROT_RIGHT, O.ROT_LEFT):
        back = O.rotate(O.rotate(V, rot, k), rot, k) / k   # (V B) B / k = V
        np.testing.assert_array_equal(back, V)
    np.testing.assert_array_equal(O.rotate(O.rotate(V, O.ROT_BOTH, k), O.ROT_BOTH, k) / k**2, V)


def test_rotation_special_blocks():
    k = 16
    c = 3.0
    V = np.zeros((1, 2 * k))
    V[0, :k] = c                 # constant block -> c*k*e0
    V[0, k + 5] = 1.0            # one-hot e_5 -> row 5 of H_k (outlier spread over the block)
    R = O.rotate(V, O.ROT_RIGHT, k)
    expect0 = np.zeros(k)
    expect0[0] = c * k
    np.testing.assert_array_equal(R[0, :k], expect0)
    np.testing.assert_array_equal(R[0, k:], scipy.linalg.hadamard(k)[5])
    np.testing.assert_array_equal(O.rotate(V, O.ROT_RIGHT, 1), V)   # k = 1: identity


def test_rotation_linearity_and_left_golden(golden):
    rng = np.random.default_rng(3)
    A, B = rng.standard_normal((8, 16)), rng.standard_normal((8, 16))
    for rot in (O.ROT_RIGHT, O.ROT_LEFT, O.ROT_BOTH):
        np.testing.assert_allclose(O.rotate(2 * A - 3 * B, rot, 4),
                                   2 * O.rotate(A, rot, 4) - 3 * O.rotate(B, rot, 4),
                                   atol=1e-12)
    ex = golden["left_rotation_k2"]
    np.testing.assert_array_equal(O.rotate(np.array(ex["g"], float), O.ROT_LEFT, ex["k"]),
                                  np.array(ex["bg"], float))


def test_rotation_rejects_misaligned():
    with pytest.raises(ValueError):
        O.rotate(np.zeros((4, 12)), O.ROT_RIGHT, 8)
    with pytest.raises(ValueError):
        O.rotate(np.zeros((12, 8)), O.ROT_LEFT, 8)


def test_rotate_i64_matches_float():
    rng = np.random.default_rng(5)
    T = rng.integers(-2**30, 2**30, size=(32, 64))
    for rot in (O.ROT_RIGHT, O.ROT_LEFT, O.ROT_BOTH):
        ref = T.astype(object)
        if rot in (O.ROT_RIGHT, O.ROT_BOTH):
            ref = ref.dot(blockdiag_h(64, 16).astype(np.int64).astype(object))
        if rot in (O.ROT_LEFT, O.ROT_BOTH):
            ref = blockdiag_h(32, 16).astype(np.int64).astype(object).dot(ref)
        np.testing.assert_array_equal(O.rotate_i64(T, rot, 16), ref.astype(np.int64))


# ----------------------------------------------------------------- quantizer
def test_quantizer_golden_worked_example(golden):
    ex = golden["fwd_int8_k4"]
    X = np.array(ex["x"], float)
    W = np.array(ex["w"], float)
    qx, sx = O.quantize_tensor(X, O.ROT_RIGHT, ex["k"], 8)
    qw, sw = O.quantize_tensor(W, O.ROT_RIGHT, ex["k"], 8)
    np.testing.assert_array_equal(qx, np.array(ex["qx"]))
    np.testing.assert_array_equal(qw, np.array(ex["qw"]))
    assert sx == ex["sx"] and sw == ex["sw"]
    y = O.fwd_from_codes(qx, sx, qw, sw, ex["k"], O.HQ)
    np.testing.assert_array_equal(y, np.array(ex["y"], float))


def test_quantizer_step_golden(golden):
    ex = golden["int4_step_k2"]
    q, s = O.quantize_tensor(np.array(ex["v"], float), O.ROT_RIGHT, ex["k"], ex["bits"],
                             O.STEP, ex["step"])
    np.testing.assert_array_equal(q, np.array(ex["codes"]))
    assert s == np.float32(ex["step"])


def test_quantizer_exact_division_near_tie_golden(golden):
    """Codes are RNE of the exact quotient V/s, not of V times a rounded reciprocal: the
    hand-derived case has s = 3 and exact midpoints that fp32(1/3) would push up."""
    g = golden["near_tie_exact_division_k2"]
    X = np.array(g["x"], dtype=np.float64)
    R = O.rotate(X, O.ROT_RIGHT, g["k"])
    np.testing.assert_array_equal(R, np.array(g["xb"], dtype=np.float64))
    q, s = O.quantize_tensor(X, O.ROT_RIGHT, g["k"], g["bits"])
    assert s == np.float32(g["s"])
    np.testing.assert_array_equal(q, np.array(g["qx"]))
    sc = g["step_case"]
    v = np.array(sc["v"], dtype=np.float64)[None, :]
    q, s = O.quantize_tensor(v, O.ROT_NONE, 1, sc["bits"], O.STEP, sc["step"])
    np.testing.assert_array_equal(q[0], np.array(sc["codes"]))


def test_absmax_scale_correctly_rounded():
    """s = a/Qp rounded once to fp32, checked against exact Fractions on values whose
    quotient lands near an fp32 midpoint (where rounding through double could slip)."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    for _ in range(300):
        f = np.float32(rng.uniform(0.5, 2.0)) * np.float32(2.0 ** rng.integers(-20, 20))
        up = np.nextafter(f, np.float32(np.inf))
        mid = (Fraction(float(f)) + Fraction(float(up))) / 2
        qp = int(rng.choice([7, 127]))
        a = float(mid * qp)   # the double nearest a midpoint times Qp
        s = O.absmax_scale(np.array([[a, -a / 3]]), qp)
        exact = Fraction(a) / qp
        cands = [f, up, np.nextafter(f, np.float32(0)), np.nextafter(up, np.float32(np.inf))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact),
                                         int(np.array(c).view(np.uint32)) & 1))
        assert s == best, (a, qp, s, best)


def test_quantizer_ties_to_even():
    v = np.array([2.5, 3.5, -2.5, 0.5, -0.5, 1.5, 126.5, -126.5])
    q = O.quantize(v, 1.0, 127)
    np.testing.assert_array_equal(q, [2, 4, -2, 0, 0, 2, 126, -126])


@pytest.mark.parametrize("bits", [8, 4])
def test_quantizer_properties(bits):
    qp = O.qmax(bits)
    rng = np.random.default_rng(11)
    R = rng.standard_normal((64, 64)) * np.exp(rng.uniform(-3, 3, (64, 64)))
    s = O.absmax_scale(R, qp)
    q = O.quantize(R, s, qp)
    assert np.abs(q).max() <= qp
    i = np.unravel_index(np.argmax(np.abs(R)), R.shape)
    assert q[i] == np.sign(R[i]) * qp                     # arg-absmax maps to +-Qp
    err = np.abs(R - s * q.astype(np.float64))
    assert (err <= s / 2 * (1 + 1e-6) + 1e-30).all()    # RTN error bound, no clipping
    np.testing.assert_array_equal(O.quantize(-R, s, qp), -q)            # odd symmetry
    for m in (-7, 3):                                     # ABSMAX invariant to 2^m scaling
        s2 = O.absmax_scale(R * 2.0 ** m, qp)
        np.testing.assert_array_equal(O.quantize(R * 2.0 ** m, s2, qp), q)
    # the scale is a32 / Qp rounded to fp32
    assert s == np.float32(np.float64(np.float32(np.abs(R).max())) / qp)


def test_quantizer_zero_tensor_and_clipping():
    Z = np.zeros((4, 8))
    q, s = O.quantize_tensor(Z, O.ROT_RIGHT, 4, 8)
    assert s == 0 and not q.any()
    q = O.quantize(np.array([100.0, -100.0, 3.2]), 1.0, 7)   # STEP mode clips at +-Qp
    np.testing.assert_array_equal(q, [7, -7, 3])


def test_qmax():
    assert O.qmax(8) == 127 and O.qmax(4) == 7
    with pytest.raises(ValueError):
        O.qmax(6)


# ------------------------------------------------------------ integer GEMM
def test_gemm_i8_brute_force_two_loop_orders():
    rng = np.random.default_rng(9)
    A = rng.integers(-128, 128, size=(4, 8)).astype(np.int8)
    B = rng.integers(-128, 128, size=(8, 8)).astype(np.int8)
    C = O.gemm_i8(A, 8, 1, B, 8, 1, 4, 8, 8)
    ref1 = np.zeros((4, 8), dtype=np.int64)
    for m in range(4):
        for n in range(8):
            for k in range(8):
                ref1[m, n] += int(A[m, k]) * int(B[k, n])
    ref2 = np.zeros((4, 8), dtype=np.int64)
    for k in range(8):
        for m in range(4):
            for n in range(8):
                ref2[m, n] += int(A[m, k]) * int(B[k, n])
    np.testing.assert_array_equal(C, ref1)
    np.testing.assert_array_equal(C, ref2)
    # transposed-operand strides give the transposed product
    np.testing.assert_array_equal(O.gemm_i8(B, 1, 8, A, 1, 8, 8, 4, 8),
                                  B.T.astype(np.int64) @ A.T.astype(np.int64))


def test_gemm_i8_overflow_guard():
    A = np.full((1, 140000), -128, dtype=np.int8)
    with pytest.raises(OverflowError):
        O.gemm_i8(A, 140000, 1, A, 1, 140000, 1, 1, 140000)
    # 127^2 * 13824 (the largest contraction of the workloads) still fits
    A = np.full((1, 13824), 127, dtype=np.int8)
    assert O.gemm_i8(A, 13824, 1, A, 1, 13824, 1, 1, 13824)[0, 0] == 127 * 127 * 13824


# ------------------------------------------- exact product identities (4x8x8)
@pytest.mark.parametrize("k", [2, 4])
def test_product_identities_exact(k):
    """Integer inputs in [-3, 3], no quantization (codes = rotated values, scales 1): the
    rotations must cancel exactly in all three products and both variants."""
    rng = np.random.default_rng(100 + k)
    N, C, D = 4, 8, 8
    X = rng.integers(-3, 4, size=(N, C)).astype(np.float64)
    W = rng.integers(-3, 4, size=(D, C)).astype(np.float64)
    G = rng.integers(-3, 4, size=(N, D)).astype(np.float64)
    i8 = lambda a: a.astype(np.int8)
    xr = i8(O.rotate(X, O.ROT_RIGHT, k))
    wr = i8(O.rotate(W, O.ROT_RIGHT, k))
    gl = i8(O.rotate(G, O.ROT_LEFT, k))
    xb = i8(O.rotate(X, O.ROT_BOTH, k))
    # (XB)(WB)^T / k = X W^T
    np.testing.assert_array_equal(O.fwd_from_codes(xr, 1, wr, 1, k, O.HQ), X @ W.T)
    # HALO2: B_N (B_N G)(W B_C) B_C / k^2 = G W
    np.testing.assert_array_equal(O.bwd_input_from_codes(gl, 1, wr, 1, k, O.HALO2), G @ W)
    # HALO2: (B_N G)^T (B_N X B_C) B_C / k^2 = G^T X
    np.testing.assert_array_equal(O.bwd_weight_from_codes(gl, 1, xb, 1, k, O.HALO2), G.T @ X)
    # HQ: (G (W B_C)) B_C / k = G W  and  (G^T (X B_C)) B_C / k = G^T X
    np.testing.assert_array_equal(O.bwd_input_from_codes(i8(G), 1, wr, 1, k, O.HQ), G @ W)
    np.testing.assert_array_equal(O.bwd_weight_from_codes(i8(G), 1, xr, 1, k, O.HQ), G.T @ X)
    # HALO0: plain products
    np.testing.assert_array_equal(O.fwd_from_codes(i8(X), 1, i8(W), 1, k, O.HALO0), X @ W.T)
    # sampled k-aligned blocks equal the corresponding slices of the full products
    full = O.bwd_input_from_codes(gl, 1, wr, 1, k, O.HALO2)
    r0 = N - k
    blk = O.bwd_input_from_codes(gl, 1, wr, 1, k, O.HALO2, row_block=(r0, k), col_block=(k, k))
    np.testing.assert_array_equal(blk, full[r0:r0 + k, k:2 * k])
    full = O.bwd_weight_from_codes(gl, 1, xb, 1, k, O.HALO2)
    blk = O.bwd_weight_from_codes(gl, 1, xb, 1, k, O.HALO2, row_block=(2, 3), col_block=(k, k))
    np.testing.assert_array_equal(blk, full[2:5, k:2 * k])


def test_brute_force_pipeline_tiny():
    """Whole HQ pipeline on 4x8x8 vs an independent brute-force evaluation in Python
    integers/fractions built from scipy's H (rotation, scale, RNE, product, dequant)."""
    from fractions import Fraction
    k, N, C, D = 4, 4, 8, 8
    rng = np.random.default_rng(77)
    X = rng.standard_normal((N, C)).astype(np.float32).astype(np.float64)
    W = rng.standard_normal((D, C)).astype(np.float32).astype(np.float64)
    out = O.linear(X, W, None, k, 8, O.HQ, passes=("fwd",))
    Hb = blockdiag_h(C, k)
    xr = [[sum(Fraction(X[i, t]) * int(Hb[t, j]) for t in range(C)) for j in range(C)]
          for i in range(N)]
    wr = [[sum(Fraction(W[i, t]) * int(Hb[t, j]) for t in range(C)) for j in range(C)]
          for i in range(D)]

    def f32_nearest(q):
        """Correctly rounded fp32 value of the Fraction q >= 0, by brute force over the
        neighbours of a first guess (ties to the even significand)."""
        f0 = np.float32(float(q))
        cands = [np.nextafter(f0, np.float32(-1)), f0, np.nextafter(f0, np.float32(np.inf))]
        return min(cands, key=lambda f: (abs(Fraction(float(f)) - q),
                                         int(np.array(f).view(np.uint32)) & 1))

    def codes(R):
        a = max(abs(v) for row in R for v in row)          # exact max |R|
        s = f32_nearest(a / 127)                           # s = a / Qp, one fp32 rounding
        q = [[int(np.clip(round(v / Fraction(float(s))), -127, 127)) for v in row]
             for row in R]                                 # RNE of the exact quotient
        return np.array(q), s

    qx, sx = codes(xr)
    qw, sw = codes(wr)
    np.testing.assert_array_equal(out["qx"], qx)   # Python round() on Fraction is RNE
    np.testing.assert_array_equal(out["qw"], qw)
    assert out["sx"] == sx and out["sw"] == sw
    y = [[float(Fraction(int(qx[i] @ qw[j])) * Fraction(float(sx)) * Fraction(float(sw)) / k)
          for j in range(D)] for i in range(N)]
    np.testing.assert_allclose(out["y"], np.array(y), rtol=1e-15, atol=0)


# ------------------------------------------------ grid-aligned end-to-end pin
@pytest.mark.parametrize("bits,k", [(8, 16), (8, 32), (4, 16)])
def test_grid_aligned_end_to_end_exact(bits, k):
    """X = A B_C / k with integer A (max |A| = Qp): rotate -> absmax -> quantize returns A with
    s = 1 exactly, and Y = A Bm^T / k = X W^T exactly (a textbook product)."""
    qp = O.qmax(bits)
    rng = np.random.default_rng(bits * 1000 + k)
    N, C, D = 2 * k, 4 * k, 3 * k
    A = rng.integers(-qp, qp + 1, size=(N, C))
    Bm = rng.integers(-qp, qp + 1, size=(D, C))
    A[0, 0], Bm[1, 2] = qp, -qp
    Hc = blockdiag_h(C, k)
    X, W = A @ Hc / k, Bm @ Hc / k
    out = O.linear(X, W, None, k, bits, O.HQ, passes=("fwd",))
    np.testing.assert_array_equal(out["qx"], A)
    np.testing.assert_array_equal(out["qw"], Bm)
    assert out["sx"] == 1.0 and out["sw"] == 1.0
    np.testing.assert_array_equal(out["y"], X @ W.T)


def test_grid_aligned_halo2_backward_exact():
    """HALO2 backward: with G = B_N Ag / k and X = B_N Axt B_C / k^2 (integer Ag, Axt with
    max = Qp), the codes are Ag and Axt exactly and dX = G W, dW = G^T X exactly."""
    k, qp = 16, 127
    N, C, D = 2 * k, 2 * k, 3 * k
    rng = np.random.default_rng(5)
    Ag = rng.integers(-qp, qp + 1, size=(N, D))
    Axt = rng.integers(-qp, qp + 1, size=(N, C))
    Aw = rng.integers(-qp, qp + 1, size=(D, C))
    Ag[0, 0] = Axt[0, 0] = Aw[0, 0] = qp
    Hn, Hc = blockdiag_h(N, k), blockdiag_h(C, k)
    G = Hn @ Ag / k
    X = Hn @ Axt @ Hc / k ** 2
    W = Aw @ Hc / k
    qg, sg = O.quantize_g(G, k, 8, O.HALO2)
    qw, sw = O.quantize_w(W, k, 8, O.HALO2)
    _, _, qxt, sxt = O.quantize_x(X, k, 8, O.HALO2)
    np.testing.assert_array_equal(qg, Ag)
    np.testing.assert_array_equal(qxt, Axt)
    np.testing.assert_array_equal(qw, Aw)
    assert sg == sw == sxt == 1.0
    np.testing.assert_array_equal(O.bwd_input_from_codes(qg, sg, qw, sw, k, O.HALO2), G @ W)
    np.testing.assert_array_equal(O.bwd_weight_from_codes(qg, sg, qxt, sxt, k, O.HALO2), G.T @ X)


# ------------------------------------------------------ derived error bound
@pytest.mark.parametrize("variant", [O.HQ, O.HALO0])
def test_fwd_error_bound(variant):
    """|Yhat - X W^T| <= (|e_x| |wr| + |xr| |e_w| + |e_x| |e_w|) / k per element, with
    |e| <= s/2 elementwise (round-to-nearest, absmax never clips)."""
    k = 32
    rng = np.random.default_rng(21)
    N, C, D = 64, 256, 96
    X = rng.standard_normal((N, C))
    X[:, [3, 77]] *= 50
    W = rng.standard_normal((D, C)) * 0.02
    out = O.linear(X, W, None, k, 8, variant, passes=("fwd",))
    kk = k if variant == O.HQ else 1
    Hc = blockdiag_h(C, kk)
    xr, wr = X @ Hc, W @ Hc
    ex = out["sx"] / 2 * np.sqrt(C) * (1 + 1e-6)
    ew = out["sw"] / 2 * np.sqrt(C) * (1 + 1e-6)
    bound = (ex * np.linalg.norm(wr, axis=1)[None, :] +
             np.linalg.norm(xr, axis=1)[:, None] * ew + ex * ew) / kk
    assert (np.abs(out["y"] - X @ W.T) <= bound).all()


def test_rotation_reduces_error_with_outliers():
    """Direction check (qualitative claim of both pages): with outlier channels, the rotated
    quantizer's product error is smaller than the unrotated one's."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((128, 512))
    X[:, [5, 100, 300, 411]] *= 50
    W = rng.standard_normal((256, 512)) * 0.02
    ref = X @ W.T
    e_hq = np.linalg.norm(O.linear(X, W, None, 32, 8, O.HQ, passes=("fwd",))["y"] - ref)
    e_h0 = np.linalg.norm(O.linear(X, W, None, 32, 8, O.HALO0, passes=("fwd",))["y"] - ref)
    assert e_hq < 0.5 * e_h0


def test_halo2_token_rotation_helps_heavy_rows():
    """Direction check (HALO page ablation: left rotation of output gradients helps): when a
    few token rows of dY are large, HALO2's dX error is below HQ's."""
    rng = np.random.default_rng(41)
    N, C, D, k = 256, 128, 128, 32
    X = rng.standard_normal((N, C))
    W = rng.standard_normal((D, C)) * 0.02
    G = rng.standard_normal((N, D)) * 1e-3
    G[[3, 90, 200]] *= 300
    ref = G @ W
    e2 = np.linalg.norm(O.linear(X, W, G, k, 8, O.HALO2, passes=("dx",))["dx"] - ref)
    e1 = np.linalg.norm(O.linear(X, W, G, k, 8, O.HQ, passes=("dx",))["dx"] - ref)
    assert e2 < e1
