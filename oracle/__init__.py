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
LIB_PATH = os.path.join(HERE, "libhq_oracle.so")

F32, F16, BF16 = 0, 1, 2
ROT_NONE, ROT_RIGHT, ROT_LEFT, ROT_BOTH = 0, 1, 2, 3
HALO0, HQ, HALO2 = 0, 1, 2
ABSMAX, STEP = 0, 1

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
    lib.hqo_dequant.argtypes = [vp, i64, f32, f32, i32, vp]
    lib.hqo_dequant.restype = None
    lib.hqo_round.argtypes = [vp, i64, i32, vp]
    lib.hqo_round.restype = i32
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def qmax(bits):
    """Symmetric grid bound: 127 for INT8, 7 for the INT4 range (INT4 page, §3.1)."""
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
    return np.float32(_load().hqo_absmax_scale(_p(R), R.size, qp))


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


def dequant(T, s_a, s_b, k_pow_e):
    T = np.ascontiguousarray(T, dtype=np.int64)
    out = np.empty(T.shape, dtype=np.float64)
    _load().hqo_dequant(_p(T), T.size, float(np.float32(s_a)), float(np.float32(s_b)),
                        int(k_pow_e), _p(out))
    return out


def round_to(vals, dtype):
    """RNE rounding of doubles to fp32 (float32 array) or fp16/bf16 (uint16 bit arrays)."""
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    out = np.empty(vals.shape, dtype=np.float32 if dtype == F32 else np.uint16)
    if _load().hqo_round(_p(vals), vals.size, dtype, _p(out)) != 0:
        raise ValueError("bad dtype")
    return out


# ------------------------------------------------------------ composed steps
def quantize_tensor(V, rot, k, bits, mode=ABSMAX, step=None):
    """Rotate -> tensor-wise scale -> codes. V is float64 (already decoded).
    Returns (codes int8, scale float32)."""
    qp = qmax(bits)
    R = rotate(V, rot, k)
    if mode == ABSMAX:
        s = absmax_scale(R, qp)
    elif mode == STEP:
        if step is None:
            raise ValueError("STEP mode needs a step")
        s = np.float32(step)
    else:
        raise ValueError("bad scale mode")
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


def quantize_x(X, k, bits, variant, mode=ABSMAX, step=None, step_xt=None):
    """Forward-pass codes of X: qX (forward operand) and, for the weight gradient, the codes
    of X in the rotation that product needs (qXt under HALO2, qX otherwise)."""
    rx, _, rxt = _rots(variant)
    qx, sx = quantize_tensor(X, rx, k, bits, mode, step)
    if rxt == rx:
        return qx, sx, qx, sx
    qxt, sxt = quantize_tensor(X, rxt, k, bits, mode, step if step_xt is None else step_xt)
    return qx, sx, qxt, sxt


def quantize_w(W, k, bits, variant, mode=ABSMAX, step=None):
    rx, _, _ = _rots(variant)
    return quantize_tensor(W, rx, k, bits, mode, step)


def quantize_g(G, k, bits, variant, mode=ABSMAX, step=None):
    _, rg, _ = _rots(variant)
    return quantize_tensor(G, rg, k, bits, mode, step)


def fwd_from_codes(qx, sx, qw, sw, k, variant, rows=None, cols=None):
    """Y[rows][cols] = (qX qW^T) sX sW / k^e in double. rows/cols: optional index ranges
    (slices) for a sampled block."""
    e = 0 if variant == HALO0 else 1
    rows = slice(None) if rows is None else rows
    cols = slice(None) if cols is None else cols
    A = np.ascontiguousarray(qx[rows])
    B = np.ascontiguousarray(qw[cols])
    M, K = A.shape
    N = B.shape[0]
    T = gemm_i8(A, K, 1, B, 1, K, M, N, K)
    return dequant(T, sx, sw, k ** e)


def bwd_input_from_codes(qg, sg, qw, sw, k, variant, row_block=None, col_block=None):
    """dX = [B_N] (qG qW) [B_C] sG sW / k^e in double. row_block/col_block: optional
    (start, length) ranges aligned to k for a sampled block (the inverse rotations only
    mix within k-blocks, so an aligned block is self-contained)."""
    N, D = qg.shape
    C = qw.shape[1]
    r0, rl = (0, N) if row_block is None else row_block
    c0, cl = (0, C) if col_block is None else col_block
    A = np.ascontiguousarray(qg[r0:r0 + rl])
    Bm = np.ascontiguousarray(qw[:, c0:c0 + cl])
    T = gemm_i8(A, D, 1, Bm, cl, 1, rl, cl, D)
    if variant == HALO2:
        T = rotate_i64(T, ROT_BOTH, k)
        e = 2
    elif variant == HQ:
        T = rotate_i64(T, ROT_RIGHT, k)
        e = 1
    else:
        e = 0
    return dequant(T, sg, sw, k ** e)


def bwd_weight_from_codes(qg, sg, qxt, sxt, k, variant, row_block=None, col_block=None):
    """dW = (qG^T qXt) [B_C] sG sXt / k^e in double (qXt = Q(B_N X B_C) under HALO2,
    qX = Q(X B_C) under HQ, Q(X) under HALO0)."""
    N, D = qg.shape
    C = qxt.shape[1]
    r0, rl = (0, D) if row_block is None else row_block
    c0, cl = (0, C) if col_block is None else col_block
    A = np.ascontiguousarray(qg[:, r0:r0 + rl])   # N x rl, contraction over tokens
    Bm = np.ascontiguousarray(qxt[:, c0:c0 + cl])  # N x cl
    T = gemm_i8(A, 1, rl, Bm, cl, 1, rl, cl, N)
    if variant == HALO2:
        T = rotate_i64(T, ROT_RIGHT, k)
        e = 2
    elif variant == HQ:
        T = rotate_i64(T, ROT_RIGHT, k)
        e = 1
    else:
        e = 0
    return dequant(T, sg, sxt, k ** e)


def linear(X, W, dY, k, bits, variant, mode=ABSMAX, steps=None, passes=("fwd", "dx", "dw")):
    """Whole linear layer from decoded float64 inputs. steps: dict with 'x', 'w', 'g' (and
    'xt') steps for STEP mode. Returns a dict of codes, scales and double outputs."""
    steps = steps or {}
    out = {}
    qx, sx, qxt, sxt = quantize_x(X, k, bits, variant, mode, steps.get("x"), steps.get("xt"))
    qw, sw = quantize_w(W, k, bits, variant, mode, steps.get("w"))
    out.update(qx=qx, sx=sx, qxt=qxt, sxt=sxt, qw=qw, sw=sw)
    if "fwd" in passes:
        out["y"] = fwd_from_codes(qx, sx, qw, sw, k, variant)
    if dY is not None and ("dx" in passes or "dw" in passes):
        qg, sg = quantize_g(dY, k, bits, variant, mode, steps.get("g"))
        out.update(qg=qg, sg=sg)
        if "dx" in passes:
            out["dx"] = bwd_input_from_codes(qg, sg, qw, sw, k, variant)
        if "dw" in passes:
            out["dw"] = bwd_weight_from_codes(qg, sg, qxt, sxt, k, variant)
    return out
