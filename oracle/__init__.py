"""CPU oracle for the Hadamard-quantized linear-layer matmul (HQ-MM).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU-baseline leg of
the benchmark, never by the product path. It shares no code with the HIP library.

The arithmetic lives in ``hq_oracle.c`` (explicit Sylvester matrix, dense rotations, scalar
quantizer, triple-loop int64 GEMM, exact int64 inverse rotations, double dequantization).
This module loads it with ctypes and composes the steps into the three products of a linear
layer, in the order the pages give them:

  "Training Transformers with 4-bit Integers", §3.1 (learned-step quantizer, Q_N = Q_P = 7,
  INT32 product dequantized), §3.3 (block-diagonal H_k, inverse-transform cancellation), §4
  (backward reuses forward-quantized activations and weights), §A.6 (HQ-MM stages);
  "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs", Approach (right rotations
  in forward, left rotation on output gradients in backward = HALO-2, tensor-wise scales,
  reuse of quantized rotated tensors).

Code formats: INT (integers on [-Qp, Qp], Qp = 127 or 7), E4M3 (FP8 codes, the HALO
page's lower-precision variants: s = max|R| / 448, nearest E4M3 value of R / s, ties to even,
saturating; products exact in int64 units of 2^-18), and E2M3 / E3M2 (FP6 codes, the same
page's FP6 variants: s = max|R| / 7.5 or / 28, nearest FP6 value, ties to even, saturating;
stored as the E4M3 bytes of their values, so the FP8 product and decode serve them).

Variants (names follow the HALO page):
  HALO0: no rotation.
  HQ   : X, W rotated on the right; dY quantized unrotated; backward reuses qW and qX.
  HALO2: as HQ, plus the token-axis (left) rotation of dY; the weight gradient contracts over
         tokens against Q(B_N X B_C), so the token rotation cancels inside that product:
           Y  = (qX qW^T) sX sW / k
           dX = B_N (qG qW) B_C sG sW / k^2,            qG  = Q(B_N dY)
           dW = (qG^T qXt) B_C sG sXt / k^2,            qXt = Q(B_N X B_C)
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# HQ_ORACLE_LIB names another build of the same source (the sanitizer test's)
LIB_PATH = os.environ.get("HQ_ORACLE_LIB") or os.path.join(HERE, "libhq_oracle.so")

F32, F16, BF16 = 0, 1, 2
ROT_NONE, ROT_RIGHT, ROT_LEFT, ROT_BOTH = 0, 1, 2, 3
HALO0, HQ, HALO2 = 0, 1, 2
ABSMAX, STEP = 0, 1
INT, E4M3 = 0, 1          # code formats: integers on [-Qp, Qp], or FP8 E4M3 values
E2M3, E3M2 = 2, 3         # FP6 code formats (stored as the E4M3 bytes of their values)
FLOAT_FORMATS = (E4M3, E2M3, E3M2)
E4M3_MAX = 448            # largest finite E4M3 value: the grid bound of the FP8 format
E4M3_UNIT_EXP = 18        # an FP8 product is an integer number of 2^-18

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    lib.hqo_version.restype = i32
    lib.hqo_threads.restype = i32
    lib.hqo_hadamard.argtypes = [i32, vp]
    lib.hqo_hadamard.restype = i32
    lib.hqo_decode.argtypes = [vp, i32, i64, vp]
    lib.hqo_decode.restype = i32
    lib.hqo_rotate.argtypes = [vp, i64, i64, i32, i32, vp]
    lib.hqo_rotate.restype = i32
    lib.hqo_absmax_scale.argtypes = [vp, i64, i32]
    lib.hqo_absmax_scale.restype = f32
    lib.hqo_quantize.argtypes = [vp, i64, f32, i32, vp]
    lib.hqo_quantize.restype = i32
    lib.hqo_gemm_i8.argtypes = [vp, i64, i64, vp, i64, i64, i64, i64, i64, vp]
    lib.hqo_gemm_i8.restype = i32
    lib.hqo_rotate_i64.argtypes = [vp, i64, i64, i32, i32, vp]
    lib.hqo_rotate_i64.restype = i32
    lib.hqo_dequant.argtypes = [vp, i64, f32, f32, ctypes.c_double, vp]
    lib.hqo_dequant.restype = None
    lib.hqo_round.argtypes = [vp, i64, i32, vp]
    lib.hqo_round.restype = i32
    lib.hqo_decode_e4m3.argtypes = [vp, i64, vp]
    lib.hqo_decode_e4m3.restype = None
    lib.hqo_quantize_e4m3.argtypes = [vp, i64, f32, vp]
    lib.hqo_quantize_e4m3.restype = i32
    lib.hqo_gemm_f8.argtypes = [vp, i64, i64, vp, i64, i64, i64, i64, i64, vp]
    lib.hqo_gemm_f8.restype = i32
    lib.hqo_absmax_scale_d.argtypes = [vp, i64, ctypes.c_double]
    lib.hqo_absmax_scale_d.restype = f32
    lib.hqo_fp6_max.argtypes = [i32]
    lib.hqo_fp6_max.restype = ctypes.c_double
    lib.hqo_quantize_fp6.argtypes = [vp, i64, f32, i32, vp]
    lib.hqo_quantize_fp6.restype = i32
    _lib = lib
    return lib


def threads():
    """OpenMP threads the oracle's loops run on."""
    return int(_load().hqo_threads())


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def qmax(bits, fmt=INT):
    """Symmetric grid bound: 127 for INT8, 7 for the INT4 range (INT4 page, §3.1), 448 for
    FP8 E4M3 codes, 7.5 / 28 for FP6 E2M3 / E3M2 codes (the largest value of each format)."""
    if fmt == E4M3:
        if bits != 8:
            raise ValueError("E4M3 codes are 8 bits")
        return E4M3_MAX
    if fmt in (E2M3, E3M2):
        if bits != 6:
            raise ValueError("FP6 codes are 6 bits")
        return fp6_max(fmt)
    if bits == 8:
        return 127
    if bits == 4:
        return 7
    raise ValueError("bits must be 4 or 8")


# ---------------------------------------------------------------- single steps
def hadamard(k):
    H = np.empty((k, k), dtype=np.int8)
    if _load().hqo_hadamard(k, _p(H)) != 0:
        raise ValueError("unsupported k=%r" % (k,))
    return H


def decode(src, dtype):
    src = np.ascontiguousarray(src)
    out = np.empty(src.shape, dtype=np.float64)
    if _load().hqo_decode(_p(src), dtype, src.size, _p(out)) != 0:
        raise ValueError("bad dtype")
    return out


def rotate(V, rot, k):
    V = np.ascontiguousarray(V, dtype=np.float64)
    rows, cols = V.shape
    R = np.empty_like(V)
    if _load().hqo_rotate(_p(V), rows, cols, rot, k, _p(R)) != 0:
        raise ValueError("rotate: bad arguments")
    return R


def absmax_scale(R, qp):
    R = np.ascontiguousarray(R, dtype=np.float64)
    if float(qp) != int(qp):   # a grid bound that is not an integer (7.5 for E2M3)
        return np.float32(_load().hqo_absmax_scale_d(_p(R), R.size, float(qp)))
    return np.float32(_load().hqo_absmax_scale(_p(R), R.size, int(qp)))


def fp6_max(fmt):
    """Largest value of an FP6 format (E2M3 or E3M2)."""
    v = _load().hqo_fp6_max(fmt)
    if v < 0:
        raise ValueError("not an FP6 format")
    return v


def quantize(R, scale, qp):
    R = np.ascontiguousarray(R, dtype=np.float64)
    q = np.empty(R.shape, dtype=np.int8)
    _load().hqo_quantize(_p(R), R.size, float(np.float32(scale)), qp, _p(q))
    return q


def gemm_i8(A, sam, sak, B, sbk, sbn, M, N, K):
    """C[m, n] = sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn], int64; raises on int32 overflow."""
    A = np.ascontiguousarray(A, dtype=np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    C = np.empty((M, N), dtype=np.int64)
    if _load().hqo_gemm_i8(_p(A), sam, sak, _p(B), sbk, sbn, M, N, K, _p(C)) != 0:
        raise OverflowError("integer product leaves the int32 range")
    return C


def rotate_i64(T, rot, k):
    T = np.ascontiguousarray(T, dtype=np.int64)
    rows, cols = T.shape
    R = np.empty_like(T)
    if _load().hqo_rotate_i64(_p(T), rows, cols, rot, k, _p(R)) != 0:
        raise ValueError("rotate_i64: bad arguments")
    return R


def dequant(T, s_a, s_b, k_pow_e, fmt=INT):
    """T * s_a * s_b / k^e (FP8 sums are in units of 2^-18: that factor is applied too)."""
    T = np.ascontiguousarray(T, dtype=np.int64)
    out = np.empty(T.shape, dtype=np.float64)
    div = float(k_pow_e) * (2.0 ** E4M3_UNIT_EXP if fmt in FLOAT_FORMATS else 1.0)
    _load().hqo_dequant(_p(T), T.size, float(np.float32(s_a)), float(np.float32(s_b)), div,
                        _p(out))
    return out


def decode_e4m3(q):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, dtype=np.float64)
    _load().hqo_decode_e4m3(_p(q), q.size, _p(out))
    return out


def quantize_e4m3(R, scale):
    """E4M3 codes (uint8) nearest to R / scale, ties to even, saturating at +-448."""
    R = np.ascontiguousarray(R, dtype=np.float64)
    q = np.empty(R.shape, dtype=np.uint8)
    _load().hqo_quantize_e4m3(_p(R), R.size, float(np.float32(scale)), _p(q))
    return q


def quantize_fp6(R, scale, fmt):
    """FP6 codes (E2M3 or E3M2) nearest to R / scale, ties to even, saturating at the largest
    value, as the uint8 E4M3 bytes of their values."""
    R = np.ascontiguousarray(R, dtype=np.float64)
    q = np.empty(R.shape, dtype=np.uint8)
    if _load().hqo_quantize_fp6(_p(R), R.size, float(np.float32(scale)), fmt, _p(q)) != 0:
        raise ValueError("not an FP6 format")
    return q


def gemm_f8(A, sam, sak, B, sbk, sbn, M, N, K):
    """Exact product of E4M3 code matrices in int64 units of 2^-18 (same index maps as
    gemm_i8)."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    C = np.empty((M, N), dtype=np.int64)
    _load().hqo_gemm_f8(_p(A), sam, sak, _p(B), sbk, sbn, M, N, K, _p(C))
    return C


def _gemm(fmt, *args):
    return gemm_f8(*args) if fmt in FLOAT_FORMATS else gemm_i8(*args)


def round_to(vals, dtype):
    """RNE rounding of doubles to fp32 (float32 array) or fp16/bf16 (uint16 bit arrays)."""
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    out = np.empty(vals.shape, dtype=np.float32 if dtype == F32 else np.uint16)
    if _load().hqo_round(_p(vals), vals.size, dtype, _p(out)) != 0:
        raise ValueError("bad dtype")
    return out


# ------------------------------------------------------------ composed steps
def quantize_tensor(V, rot, k, bits, mode=ABSMAX, step=None, fmt=INT):
    """Rotate -> tensor-wise scale -> codes. V is float64 (already decoded).
    Returns (codes: int8, or uint8 E4M3 bytes for the float formats; scale: float32)."""
    qp = qmax(bits, fmt)
    R = rotate(V, rot, k)
    if mode == ABSMAX:
        s = absmax_scale(R, qp)
    elif mode == STEP:
        if step is None:
            raise ValueError("STEP mode needs a step")
        s = np.float32(step)
    else:
        raise ValueError("bad scale mode")
    if fmt == E4M3:
        return quantize_e4m3(R, s), s
    if fmt in (E2M3, E3M2):
        return quantize_fp6(R, s, fmt), s
    return quantize(R, s, qp), s


def _rots(variant):
    """(rotation of X/W codes, rotation of dY codes, rotation of the dW right operand)."""
    if variant == HALO0:
        return ROT_NONE, ROT_NONE, ROT_NONE
    if variant == HQ:
        return ROT_RIGHT, ROT_NONE, ROT_RIGHT
    if variant == HALO2:
        return ROT_RIGHT, ROT_LEFT, ROT_BOTH
    raise ValueError("bad variant")


def quantize_x(X, k, bits, variant, mode=ABSMAX, step=None, step_xt=None, fmt=INT):
    """Forward-pass codes of X: qX (forward operand) and, for the weight gradient, the codes
    of X in the rotation that product needs (qXt under HALO2, qX otherwise)."""
    rx, _, rxt = _rots(variant)
    qx, sx = quantize_tensor(X, rx, k, bits, mode, step, fmt)
    if rxt == rx:
        return qx, sx, qx, sx
    qxt, sxt = quantize_tensor(X, rxt, k, bits, mode, step if step_xt is None else step_xt, fmt)
    return qx, sx, qxt, sxt


def quantize_w(W, k, bits, variant, mode=ABSMAX, step=None, fmt=INT):
    rx, _, _ = _rots(variant)
    return quantize_tensor(W, rx, k, bits, mode, step, fmt)


def quantize_g(G, k, bits, variant, mode=ABSMAX, step=None, fmt=INT):
    _, rg, _ = _rots(variant)
    return quantize_tensor(G, rg, k, bits, mode, step, fmt)


def fwd_from_codes(qx, sx, qw, sw, k, variant, rows=None, cols=None, fmt=INT):
    """Y[rows][cols] = (qX qW^T) sX sW / k^e in double. rows/cols: optional index ranges
    (slices) for a sampled block."""
    e = 0 if variant == HALO0 else 1
    rows = slice(None) if rows is None else rows
    cols = slice(None) if cols is None else cols
    A = np.ascontiguousarray(qx[rows])
    B = np.ascontiguousarray(qw[cols])
    M, K = A.shape
    N = B.shape[0]
    T = _gemm(fmt, A, K, 1, B, 1, K, M, N, K)
    return dequant(T, sx, sw, k ** e, fmt)


def bwd_input_from_codes(qg, sg, qw, sw, k, variant, row_block=None, col_block=None, fmt=INT):
    """dX = [B_N] (qG qW) [B_C] sG sW / k^e in double. row_block/col_block: optional
    (start, length) ranges aligned to k for a sampled block (the inverse rotations only
    mix within k-blocks, so an aligned block is self-contained)."""
    N, D = qg.shape
    C = qw.shape[1]
    r0, rl = (0, N) if row_block is None else row_block
    c0, cl = (0, C) if col_block is None else col_block
    A = np.ascontiguousarray(qg[r0:r0 + rl])
    Bm = np.ascontiguousarray(qw[:, c0:c0 + cl])
    T = _gemm(fmt, A, D, 1, Bm, cl, 1, rl, cl, D)
    if variant == HALO2:
        T = rotate_i64(T, ROT_BOTH, k)
        e = 2
    elif variant == HQ:
        T = rotate_i64(T, ROT_RIGHT, k)
        e = 1
    else:
        e = 0
    return dequant(T, sg, sw, k ** e, fmt)


def bwd_weight_from_codes(qg, sg, qxt, sxt, k, variant, row_block=None, col_block=None, fmt=INT):
    """dW = (qG^T qXt) [B_C] sG sXt / k^e in double (qXt = Q(B_N X B_C) under HALO2,
    qX = Q(X B_C) under HQ, Q(X) under HALO0)."""
    N, D = qg.shape
    C = qxt.shape[1]
    r0, rl = (0, D) if row_block is None else row_block
    c0, cl = (0, C) if col_block is None else col_block
    A = np.ascontiguousarray(qg[:, r0:r0 + rl])   # N x rl, contraction over tokens
    Bm = np.ascontiguousarray(qxt[:, c0:c0 + cl])  # N x cl
    T = _gemm(fmt, A, 1, rl, Bm, cl, 1, rl, cl, N)
    if variant == HALO2:
        T = rotate_i64(T, ROT_RIGHT, k)
        e = 2
    elif variant == HQ:
        T = rotate_i64(T, ROT_RIGHT, k)
        e = 1
    else:
        e = 0
    return dequant(T, sg, sxt, k ** e, fmt)


def linear(X, W, dY, k, bits, variant, mode=ABSMAX, steps=None, passes=("fwd", "dx", "dw"),
           fmt=INT):
    """Whole linear layer from decoded float64 inputs. steps: dict with 'x', 'w', 'g' (and
    'xt') steps for STEP mode. fmt: INT codes or FP8 E4M3 codes. Returns a dict of codes,
    scales and double outputs."""
    steps = steps or {}
    out = {}
    qx, sx, qxt, sxt = quantize_x(X, k, bits, variant, mode, steps.get("x"), steps.get("xt"), fmt)
    qw, sw = quantize_w(W, k, bits, variant, mode, steps.get("w"), fmt)
    out.update(qx=qx, sx=sx, qxt=qxt, sxt=sxt, qw=qw, sw=sw)
    if "fwd" in passes:
        out["y"] = fwd_from_codes(qx, sx, qw, sw, k, variant, fmt=fmt)
    if dY is not None and ("dx" in passes or "dw" in passes):
        qg, sg = quantize_g(dY, k, bits, variant, mode, steps.get("g"), fmt)
        out.update(qg=qg, sg=sg)
        if "dx" in passes:
            out["dx"] = bwd_input_from_codes(qg, sg, qw, sw, k, variant, fmt=fmt)
        if "dw" in passes:
            out["dw"] = bwd_weight_from_codes(qg, sg, qxt, sxt, k, variant, fmt=fmt)
    return out


# ------------------------------------------------------------ batched products
def linear_batched(X, W, dY, k, bits, variant, mode=ABSMAX, steps=None,
                   passes=("fwd", "dx", "dw"), fmt=INT):
    """Batched HQ-MM ("Training Transformers with 4-bit Integers", §A.1: the batched matmuls of
    attention use the same quantizers as ordinary ones). X: batch x N x C, W: batch x D x C,
    dY: batch x N x D (float64). Each batched tensor is quantized as one tensor, stacked along
    its rows (one scale; right rotations act within rows, token blocks of k rows stay inside a
    batch since N % k == 0); batch b's products use batch b's codes. Returns stacked codes,
    scales and per-batch double outputs (batch x ... arrays)."""
    nb, N, C = X.shape
    D = W.shape[1]
    steps = steps or {}
    out = {}
    qx, sx, qxt, sxt = quantize_x(X.reshape(nb * N, C), k, bits, variant, mode, steps.get("x"),
                                  steps.get("xt"), fmt)
    qw, sw = quantize_w(W.reshape(nb * D, C), k, bits, variant, mode, steps.get("w"), fmt)
    out.update(qx=qx, sx=sx, qxt=qxt, sxt=sxt, qw=qw, sw=sw)
    xs = [slice(b * N, (b + 1) * N) for b in range(nb)]
    ws = [slice(b * D, (b + 1) * D) for b in range(nb)]
    if "fwd" in passes:
        out["y"] = np.stack([fwd_from_codes(qx[xs[b]], sx, qw[ws[b]], sw, k, variant, fmt=fmt)
                             for b in range(nb)])
    if dY is not None and ("dx" in passes or "dw" in passes):
        qg, sg = quantize_g(dY.reshape(nb * N, D), k, bits, variant, mode, steps.get("g"), fmt)
        out.update(qg=qg, sg=sg)
        if "dx" in passes:
            out["dx"] = np.stack([bwd_input_from_codes(qg[xs[b]], sg, qw[ws[b]], sw, k, variant,
                                                       fmt=fmt) for b in range(nb)])
        if "dw" in passes:
            out["dw"] = np.stack([bwd_weight_from_codes(qg[xs[b]], sg, qxt[xs[b]], sxt, k,
                                                        variant, fmt=fmt) for b in range(nb)])
    return out


# ------------------------------------------------ quantizer parameters (LSQ step machinery)
def lsq_step_derivative(R, scale, qp):
    """d v_hat / d s for v_hat = s * clamp(RNE(v / s), -Qp, Qp) with the straight-through
    rounding of learned step size quantization ("Training Transformers with 4-bit Integers",
    §3.1 learned step, §A.3 step gradients by the chain rule): q - v/s inside the grid, and
    the clipped level (+-Qp) outside it. The quotient is exact (double of an exact R over an
    fp32 s); the codes are the oracle's quantizer."""
    R = np.ascontiguousarray(R, dtype=np.float64)
    q = quantize(R, scale, qp).astype(np.float64)
    x = R / float(np.float32(scale))
    return np.where(np.abs(x) >= qp, np.sign(x) * qp, q - x)


def rotated_stats(V, G, rot, k, bits, scale, fmt=INT):
    """The three statistics of a rotated tensor R = rotation(V) that set quantizer parameters
    (INT4 page §A.3-§A.5), each the plain sum over all entries, in double:
      abs_sum  = sum |R|                                   (cold-start step)
      qerr     = sum (R - s * value(code(R)))^2              (Hadamard-size selection)
      lsq      = sum (rotation(G) / k)_i * d v_hat_i / d s   (LSQ step gradient; G the gradient
                 of the loss with respect to the unrotated tensor, so rotation(G) / k is the
                 gradient with respect to R since V = R B / k)
    lsq is None when G is None; INT codes only for lsq."""
    R = rotate(V, rot, k)
    out = {"abs_sum": float(np.sum(np.abs(R)))}
    qp = qmax(bits, fmt)
    if fmt == E4M3:
        rec = decode_e4m3(quantize_e4m3(R, scale)) * float(np.float32(scale))
    elif fmt in (E2M3, E3M2):
        rec = decode_e4m3(quantize_fp6(R, scale, fmt)) * float(np.float32(scale))
    else:
        rec = quantize(R, scale, qp).astype(np.float64) * float(np.float32(scale))
    out["qerr"] = float(np.sum((R - rec) ** 2))
    if G is not None:
        kk = k if rot != ROT_NONE else 1
        Gr = rotate(G, rot, k) / kk
        out["lsq"] = float(np.sum(Gr * lsq_step_derivative(R, scale, qp)))
    return out


def cold_start_step(V, rot, k, bits):
    """Cold-start step of a tensor (INT4 page §A.4: while steps are not yet learned, a
    heuristic sets them from the tensor; the page does not give it). Reading taken: the
    learned-step initialisation 2 * mean|R| / sqrt(Qp) of the rotated tensor, rounded once to
    fp32."""
    R = rotate(V, rot, k)
    return np.float32(2.0 * float(np.mean(np.abs(R))) / np.sqrt(qmax(bits)))


def choose_hadamard_k(X, W, candidates, bits, fmt=INT):
    """Hadamard size selection (INT4 page §A.5): the candidate k minimising the product of the
    activation and weight quantization errors, the rotated tensors standing for X and W:
    err(V, k) = ||V - s Q(V B) B / k||_F^2 = sum (R - s q)^2 / k (B B = k I), with the tensor-
    wise absmax scale of R = V B. Returns (best k, {k: (err_x, err_w)}); ties go to the earlier
    candidate."""
    errs = {}
    best = None
    for k in candidates:
        e = []
        for V in (X, W):
            R = rotate(V, ROT_RIGHT, k)
            s = absmax_scale(R, qmax(bits, fmt))
            e.append(rotated_stats(V, None, ROT_RIGHT, k, bits, s, fmt)["qerr"] / k)
        errs[k] = tuple(e)
        if best is None or e[0] * e[1] < errs[best][0] * errs[best][1]:
            best = k
    return best, errs


# ------------------------------------------------ LSS-MM: the sampled weight gradient
LSS_HI_QP = 7          # both halves of the bit split are INT4-range codes
LSS_LO_DIV = 14        # s_lo = s_hi / 14: the smallest step whose [-7, 7] covers a half step


def lss_probabilities(scores, budget):
    """Leverage-score sampling probabilities ("Training Transformers with 4-bit Integers",
    §4.2 probabilities in proportion to leverage scores, §A.2 the clamp-and-rescale
    procedure): p = (budget / sum(l)) l; while some p exceed 1, those are set to 1 and the
    others rescaled to fill what remains of the budget. Zero scores get p = 0; if the budget
    covers every nonzero score they all get 1. Double precision, sums in index order."""
    l = np.asarray(scores, dtype=np.float64)
    p = np.zeros_like(l)
    fixed = np.zeros(l.shape, dtype=bool)        # probabilities clamped to 1
    nonzero = l > 0
    while True:
        free = nonzero & ~fixed
        left = float(budget) - float(np.count_nonzero(fixed))
        if not free.any() or left <= 0:
            break
        tot = 0.0
        for v in l[free]:                        # the sum in index order
            tot += float(v)
        p[free] = (left / tot) * l[free]         # one scale factor per round
        over = free & (p > 1.0)
        if not over.any():
            break
        p[over] = 1.0
        fixed |= over
    return p


def lss_weight_gradient(G, qx, sx, k, budget, uniforms, rot=ROT_RIGHT, dw_rows=None):
    """LSS-MM for the weight gradient of the INT4-range HQ layer (INT4 page §4.2 bit splitting
    and leverage-score sampling, §A.2 probabilities, §A.3 LSS-MM stages, §A.6 INT8 data for the
    scores and K padding after sampling, §B.2 the unbiased row-sampled estimator):
      1. scores: q8 = Q(dY) on the INT8 grid (tensor-wise absmax), l_i = |q8_i| |qx_i|
         (Euclidean norms of integer rows; qx = the forward's codes of X B_C);
      2. probabilities p = lss_probabilities(l, budget); token i is kept iff u_i < p_i (the
         uniforms are an input);
      3. kept rows weighted by 1 / p_i (unbiased: E[sum m_i / p_i g_i x_i] = sum g_i x_i);
      4. bit split of the kept, weighted rows Gw: s_hi = max|Gw| / 7, hi = Q_7(Gw / s_hi),
         s_lo = s_hi / 14, lo = Q_7((Gw - s_hi hi) / s_lo); Gw ~ s_lo (14 hi + lo);
      5. dW = (14 hi + lo)^T qx_kept B_C s_lo sx / k: the two INT4 products (hi, lo) summed
         exactly as one integer product over the kept tokens, then the inverse rotation.
    dw_rows: optional index array or slice of the rows of dW to form (all by default).
    Returns a dict: scores, p, keep (indices), s_hi, s_lo, hi, lo, dw (double, D x C, or
    len(dw_rows) x C)."""
    G = np.ascontiguousarray(G, dtype=np.float64)
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    N, D = G.shape
    C = qx.shape[1]
    s8 = absmax_scale(G, 127)
    q8 = quantize(G, s8, 127).astype(np.int64)
    xi = qx.astype(np.int64)
    scores = np.sqrt((q8 * q8).sum(axis=1).astype(np.float64)) * \
        np.sqrt((xi * xi).sum(axis=1).astype(np.float64))
    p = lss_probabilities(scores, budget)
    keep = np.nonzero(np.asarray(uniforms, dtype=np.float32).astype(np.float64) < p)[0]
    out = {"scores": scores, "p": p, "keep": keep}
    Gw = G[keep] / p[keep][:, None]
    s_hi = absmax_scale(Gw, LSS_HI_QP) if keep.size else np.float32(0)
    hi = quantize(Gw, s_hi, LSS_HI_QP)
    s_lo = np.float32(float(s_hi) / LSS_LO_DIV)
    lo = quantize(Gw - float(s_hi) * hi.astype(np.float64), s_lo, LSS_HI_QP)
    out.update(s_hi=s_hi, s_lo=s_lo, hi=hi, lo=lo)
    comb = (LSS_LO_DIV * hi.astype(np.int64) + lo.astype(np.int64)).astype(np.int8)
    if dw_rows is not None:
        comb = np.ascontiguousarray(comb[:, dw_rows])
    Dr = comb.shape[1]
    xk = np.ascontiguousarray(qx[keep])
    K = keep.size
    T = gemm_i8(comb, 1, Dr, xk, C, 1, Dr, C, K) if K else np.zeros((Dr, C), dtype=np.int64)
    kk = 1
    if rot == ROT_RIGHT:
        T = rotate_i64(T, ROT_RIGHT, k)
        kk = k
    out["dw"] = dequant(T, s_lo, sx, kk)
    return out
