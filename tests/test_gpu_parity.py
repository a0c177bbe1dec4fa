"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Sizes here run in seconds on the oracle and still span several kernel tiles plus ragged
tails; the full workload sizes are covered by test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
from hadamard_rotated_precision_amd import binding as B
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

from hq_testlib import (assert_codes, assert_scale, compare_layer, host, outputs_from_gpu_codes,
                        rel_fro, rounded, run_gpu, run_oracle)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def banner(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ integer GEMM
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (256, 256, 64), (300, 257, 1040), (513, 129, 4096),
                                   (64, 700, 48), (256, 512, 0), (17, 33, 8)])
def test_gemm_i8_i32_bitexact(M, N, K):
    banner("gemm", M, N, K)
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    lda = ldb = max(16, (K + 15) // 16 * 16)
    A = np.zeros((M, lda), dtype=np.int8)
    Bt = np.zeros((N, ldb), dtype=np.int8)
    A[:, :K] = rng.integers(-128, 128, size=(M, K))
    Bt[:, :K] = rng.integers(-128, 128, size=(N, K))
    a = torch.from_numpy(A).to(DEV)
    b = torch.from_numpy(Bt).to(DEV)
    c = torch.full((M, N), 12345, dtype=torch.int32, device=DEV)
    B.check(B.hq_gemm_i8_i32(a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), M, N, K,
                             T.stream_ptr()), "gemm")
    torch.cuda.synchronize()
    ref = O.gemm_i8(A[:, :K], K, 1, Bt[:, :K], 1, K, M, N, K) if K else np.zeros((M, N), np.int64)
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("M,N,K", [(8192, 5120, 64), (4000, 5000, 48), (12288, 3072, 32)])
def test_gemm_i8_i32_wide_then_narrow(M, N, K):
    """Shapes whose 256 x 256 tile grid would leave the last round of workgroups partly filled:
    256-wide tiles cover the leading columns and a second launch of 128-wide tiles the rest
    (8192 x 5120: 4096 + 1024 columns; ragged rows and a ragged tail at 4000 x 5000). Every entry, bit for bit (the reference product is
    exact in float64 at these magnitudes)."""
    banner("gemm-tail", M, N, K)
    rng = np.random.default_rng(M + N + K)
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Bt = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    a, b = torch.from_numpy(A).to(DEV), torch.from_numpy(Bt).to(DEV)
    c = torch.full((M, N), 12345, dtype=torch.int32, device=DEV)
    B.check(B.hq_gemm_i8_i32(a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), M, N, K,
                             T.stream_ptr()), "gemm")
    torch.cuda.synchronize()
    ref = A.astype(np.float64) @ Bt.astype(np.float64).T
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.float64), ref)


def test_gemm_extremes_fit_int32():
    """All -128 / 127 operands at the largest contraction of the workloads (13824)."""
    K, M, N = 13824, 64, 64
    A = np.full((M, K), -128, dtype=np.int8)
    A[1::2] = 127
    Bt = np.full((N, K), -128, dtype=np.int8)
    a, b = torch.from_numpy(A).to(DEV), torch.from_numpy(Bt).to(DEV)
    c = torch.empty((M, N), dtype=torch.int32, device=DEV)
    B.check(B.hq_gemm_i8_i32(a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), M, N, K,
                             T.stream_ptr()), "gemm")
    torch.cuda.synchronize()
    ref = A[:, :1].astype(np.int64) * -128 * K
    np.testing.assert_array_equal(c.cpu().numpy()[:, :1], ref)


# ------------------------------------------------------------------ FWHT (exact)
@pytest.mark.parametrize("k", [1, 2, 4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("rot", [B.HQ_ROT_RIGHT, B.HQ_ROT_LEFT])
@pytest.mark.parametrize("dt", [B.HQ_F32, B.HQ_BF16, B.HQ_F16])
def test_fwht_exact_on_small_integers(k, rot, dt):
    """Small-integer inputs make every partial sum exact in fp32, so the butterfly result must
    equal the oracle's dense product with the explicit H bit for bit."""
    banner("fwht", k, rot, dt)
    rng = np.random.default_rng(k + 10 * rot + 100 * dt)
    rows = 2 * max(k, 8) if rot == B.HQ_ROT_LEFT else 37
    cols = 3 * max(k, 16) + (0 if rot == B.HQ_ROT_RIGHT else 5)
    V = rng.integers(-8, 9, size=(rows, cols)).astype(np.float32)
    bits = WL.to_dtype_bits(V.astype(np.float64), dt)
    src = T.device_tensor_from_bits(bits, dt, DEV)
    dst = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    B.check(B.hq_fwht(src.data_ptr(), dt, dst.data_ptr(), B.HQ_F32, rows, cols, rot, k,
                      T.stream_ptr()), "fwht")
    torch.cuda.synchronize()
    ref = O.rotate(V.astype(np.float64), rot, k)
    np.testing.assert_array_equal(dst.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("k", [4, 16, 64, 256])
@pytest.mark.parametrize("rot", [B.HQ_ROT_RIGHT, B.HQ_ROT_LEFT])
@pytest.mark.parametrize("dt", [B.HQ_BF16, B.HQ_F16])
@pytest.mark.parametrize("ragged", [False, True])
def test_fwht_16bit_output_exact(k, rot, dt, ragged):
    """16-bit outputs, whole aligned runs (vector stores) and partial or unaligned ones (element
    stores: rows of 8 columns at k = 4, rows of 197 columns): with small-integer inputs the fp32 sums are exact, so each output must be the exact rotation
    rounded once to the dtype (nearest even), bit for bit. At k = 256 the bf16 rounding is
    active (sums up to 2048 need 12 bits)."""
    banner("fwht16", k, rot, dt, ragged)
    rng = np.random.default_rng(7 * k + rot + 31 * dt + 5 * ragged)
    if rot == B.HQ_ROT_RIGHT:
        rows, cols = (37 if ragged else 64), 2 * k
    else:
        rows, cols = 2 * k, (3 * 64 + 5 if ragged else 3 * 64)
    V = rng.integers(-8, 9, size=(rows, cols)).astype(np.float64)
    src = torch.from_numpy(V.astype(np.float32)).to(DEV)
    dst = torch.empty((rows, cols), dtype=T.TORCH_DT[dt], device=DEV)
    B.check(B.hq_fwht(src.data_ptr(), B.HQ_F32, dst.data_ptr(), dt, rows, cols, rot, k,
                      T.stream_ptr()), "fwht")
    torch.cuda.synchronize()
    expect = WL.to_dtype_bits(O.rotate(V, rot, k), dt)
    np.testing.assert_array_equal(T.bits_of(dst), expect)


@pytest.mark.parametrize("path", [B.HQ_FWHT_AUTO, B.HQ_FWHT_BUTTERFLY, B.HQ_FWHT_MATRIX])
@pytest.mark.parametrize("k", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dt", [B.HQ_BF16, B.HQ_F16])
@pytest.mark.parametrize("rot", [B.HQ_ROT_RIGHT, B.HQ_ROT_LEFT])
def test_fwht_matrix_core_exact(rot, k, dt, path):
    """16-bit in = out on whole tiles (64 x 256 RIGHT, 256 x 64 LEFT), through each path of
    hq_fwht_path: the matrix cores (exact +-1 products, fp32 sums, back through LDS), the VALU
    butterflies, and the automatic choice. Small integers keep the sums exact, so every
    output is the exact rotation rounded once, bit for bit, whichever path runs."""
    banner("fwht-path", rot, k, dt, path)
    rng = np.random.default_rng(11 * k + dt + 3 * rot)
    rows, cols = (128, 512) if rot == B.HQ_ROT_RIGHT else (512, 192)
    V = rng.integers(-8, 9, size=(rows, cols)).astype(np.float64)
    src = T.device_tensor_from_bits(WL.to_dtype_bits(V, dt), dt, DEV)
    dst = torch.full((rows, cols), 7.0, dtype=T.TORCH_DT[dt], device=DEV)
    B.check(B.hq_fwht_path(src.data_ptr(), dt, dst.data_ptr(), dt, rows, cols, rot, k, path,
                           T.stream_ptr()), "fwht")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(T.bits_of(dst), WL.to_dtype_bits(O.rotate(V, rot, k), dt))


@pytest.mark.parametrize("which", ["src", "dst"])
@pytest.mark.parametrize("rot", [B.HQ_ROT_RIGHT, B.HQ_ROT_LEFT])
def test_fwht_unaligned_pointers(rot, which):
    """Whole tiles but a source or destination 2 bytes past a 16-byte boundary: the transform
    takes the element-access path of the VALU kernels instead of the matrix cores, with the
    same exact result."""
    banner("fwht-unaligned", rot, which)
    dt, k = B.HQ_BF16, 128
    rng = np.random.default_rng(71 + rot)
    rows, cols = (128, 512) if rot == B.HQ_ROT_RIGHT else (512, 192)
    V = rng.integers(-8, 9, size=(rows, cols)).astype(np.float64)
    bits = WL.to_dtype_bits(V, dt)
    sbuf = torch.zeros(rows * cols + 8, dtype=torch.bfloat16, device=DEV)
    dbuf = torch.zeros(rows * cols + 8, dtype=torch.bfloat16, device=DEV)
    so = 1 if which == "src" else 0
    do = 1 if which == "dst" else 0
    sbuf[so:so + rows * cols] = T.device_tensor_from_bits(bits, dt, DEV).reshape(-1)
    B.check(B.hq_fwht(sbuf[so:].data_ptr(), dt, dbuf[do:].data_ptr(), dt, rows, cols, rot, k,
                      T.stream_ptr()), "fwht")
    torch.cuda.synchronize()
    got = T.bits_of(dbuf[do:do + rows * cols].reshape(rows, cols))
    np.testing.assert_array_equal(got, WL.to_dtype_bits(O.rotate(V, rot, k), dt))


@pytest.mark.parametrize("dt", [B.HQ_BF16, B.HQ_F16])
@pytest.mark.parametrize("rot", [B.HQ_ROT_RIGHT, B.HQ_ROT_LEFT])
def test_fwht_matrix_core_random(rot, dt):
    """Normal inputs on the matrix-core transforms (k = 128, several tiles per workgroup):
    within the 16-bit rounding of the exact rotation."""
    banner("fwht-mma-random", rot, dt)
    rng = np.random.default_rng(5 + dt + 7 * rot)
    rows, cols, k = 2048, 4096, 128
    V = rng.standard_normal((rows, cols))
    bits = WL.to_dtype_bits(V, dt)
    src = T.device_tensor_from_bits(bits, dt, DEV)
    dst = torch.empty((rows, cols), dtype=T.TORCH_DT[dt], device=DEV)
    B.check(B.hq_fwht(src.data_ptr(), dt, dst.data_ptr(), dt, rows, cols, rot, k,
                      T.stream_ptr()), "fwht")
    torch.cuda.synchronize()
    ref = O.rotate(O.decode(bits, dt), rot, k)
    got = O.decode(T.bits_of(dst), dt)
    assert rel_fro(got, rounded(ref, dt)) < 1e-4
    # per element: one ulp of the dtype (the final rounding) plus the fp32 summation error of
    # the k terms, bounded by 2^-20 of the block's sum of |input| (this matters where the
    # terms cancel)
    mant, emin = (7, -126) if dt == B.HQ_BF16 else (10, -14)
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))), emin)
    a = np.abs(O.decode(bits, dt))
    if rot == B.HQ_ROT_LEFT:
        absum = np.repeat(a.reshape(rows // k, k, cols).sum(axis=1), k, axis=0)
    else:
        absum = np.repeat(a.reshape(rows, cols // k, k).sum(axis=2), k, axis=1)
    assert np.all(np.abs(got - ref) <= 2.0 ** (e - mant) + 2.0 ** -20 * absum)


@pytest.mark.parametrize("k", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dt,out", [(B.HQ_BF16, B.HQ_BF16), (B.HQ_F16, B.HQ_F16),
                                    (B.HQ_BF16, B.HQ_F32)])
@pytest.mark.parametrize("reg", ["1", "0"])
def test_fwht_left_butterfly(k, dt, out, reg, monkeypatch):
    """LEFT on the VALU butterflies, 16-bit input: at k = 16 the register kernel (a 16-row block
    of 8 columns per lane, no LDS) and, with HQ_COLS_REG=0, the LDS-staged one, which every
    larger k takes. 2048 x 1000 leaves a partial column tile at every k. Small integers: the
    exact rotation rounded once, bit for bit; normal inputs: within one unit of the output
    dtype plus the fp32 summation error."""
    monkeypatch.setenv("HQ_COLS_REG", reg)
    banner("fwht-left-butterfly", k, dt, out, reg)
    rows, cols = 2048, 1000
    rng = np.random.default_rng(13 * k + dt + 5 * out)
    for exact in (True, False):
        V = (rng.integers(-8, 9, size=(rows, cols)).astype(np.float64) if exact
             else rng.standard_normal((rows, cols)))
        bits = WL.to_dtype_bits(V, dt)
        src = T.device_tensor_from_bits(bits, dt, DEV)
        dst = torch.full((rows, cols), 7.0, dtype=T.TORCH_DT[out], device=DEV)
        B.check(B.hq_fwht_path(src.data_ptr(), dt, dst.data_ptr(), out, rows, cols,
                               B.HQ_ROT_LEFT, k, B.HQ_FWHT_BUTTERFLY, T.stream_ptr()), "fwht")
        torch.cuda.synchronize()
        ref = O.rotate(O.decode(bits, dt), O.ROT_LEFT, k)
        if exact:
            if out == B.HQ_F32:
                np.testing.assert_array_equal(dst.cpu().numpy().astype(np.float64), ref)
            else:
                np.testing.assert_array_equal(T.bits_of(dst), WL.to_dtype_bits(ref, out))
            continue
        got = O.decode(T.bits_of(dst), out)
        mant, emin = {B.HQ_BF16: (7, -126), B.HQ_F16: (10, -14), B.HQ_F32: (23, -126)}[out]
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))), emin)
        absum = np.repeat(np.abs(O.decode(bits, dt)).reshape(rows // k, k, cols).sum(axis=1), k,
                          axis=0)
        assert np.all(np.abs(got - ref) <= 2.0 ** (e - mant) + 2.0 ** -20 * absum)


def test_fwht_output_dtypes():
    rng = np.random.default_rng(3)
    V = rng.standard_normal((64, 256)).astype(np.float32)
    src = torch.from_numpy(V).to(DEV)
    ref = O.rotate(V.astype(np.float64), O.ROT_RIGHT, 64)
    for dt in (B.HQ_BF16, B.HQ_F16):
        dst = torch.empty((64, 256), dtype=T.TORCH_DT[dt], device=DEV)
        B.check(B.hq_fwht(src.data_ptr(), B.HQ_F32, dst.data_ptr(), dt, 64, 256, B.HQ_ROT_RIGHT,
                          64, T.stream_ptr()), "fwht")
        torch.cuda.synchronize()
        got = O.decode(T.bits_of(dst), dt)
        assert rel_fro(got, rounded(ref, dt)) < 1e-3


# ---------------------------------------------------------- rotate + quantize
def _rq(V_bits, dt, rows, cols, rot, k, bits, mode, step=None, codes=True, codes_t=True):
    q = T.QTensor(rows, cols, codes=codes, codes_t=codes_t)
    cfg = T.config(k, bits, mode, B.HQ_VARIANT_HQ)
    ws_bytes = B.hq_workspace_bytes(cfg, rows, cols, cols)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    src = T.device_tensor_from_bits(V_bits, dt, DEV)
    st = None if step is None else torch.tensor([step], dtype=torch.float32, device=DEV)
    B.check(B.hq_rotate_quantize(src.data_ptr(), dt, rows, cols, rot, cfg, T.ptr(st), q.st,
                                 ws.data_ptr(), ws_bytes, T.stream_ptr()), "rotate_quantize")
    torch.cuda.synchronize()
    return q


@pytest.mark.parametrize("rot,k,rows,cols", [
    (B.HQ_ROT_NONE, 1, 300, 100),
    (B.HQ_ROT_RIGHT, 16, 300, 1040),
    (B.HQ_ROT_RIGHT, 32, 77, 512),
    (B.HQ_ROT_RIGHT, 256, 129, 768),
    (B.HQ_ROT_RIGHT, 4, 33, 36),
    (B.HQ_ROT_RIGHT, 256, 128, 512),     # whole 64 x 256 tiles: the persistent kernel
    (B.HQ_ROT_RIGHT, 128, 192, 1024),
    (B.HQ_ROT_RIGHT, 64, 64, 256),
    (B.HQ_ROT_RIGHT, 16, 64, 512),       # matrix-core rotation, k = 16 and 32 blocks
    (B.HQ_ROT_RIGHT, 32, 128, 768),
    (B.HQ_ROT_NONE, 1, 64, 512),
    (B.HQ_ROT_LEFT, 256, 512, 300),
    (B.HQ_ROT_LEFT, 16, 48, 200),
    (B.HQ_ROT_LEFT, 8, 24, 100),
    (B.HQ_ROT_LEFT, 128, 256, 64),
    (B.HQ_ROT_LEFT, 256, 512, 192),      # whole 256 x 64 tiles: the persistent kernel
    (B.HQ_ROT_LEFT, 64, 768, 128),
    (B.HQ_ROT_LEFT, 2, 256, 64),
    (B.HQ_ROT_LEFT, 16, 256, 128),       # matrix-core token-axis rotation, k = 16 and 32
    (B.HQ_ROT_LEFT, 32, 512, 64),
    (B.HQ_ROT_BOTH, 256, 512, 512),
    (B.HQ_ROT_BOTH, 128, 256, 384),
    (B.HQ_ROT_BOTH, 16, 64, 48),
    (B.HQ_ROT_BOTH, 128, 256, 512),      # whole 256 x 256 tiles: matrix-core row phase
    (B.HQ_ROT_BOTH, 16, 256, 256),
    (B.HQ_ROT_BOTH, 64, 512, 768),
    (B.HQ_ROT_BOTH, 16, 2048, 4352),     # 272 items on 256 workgroups: pipelined raw loads
])
@pytest.mark.parametrize("bits,mode", [(8, B.HQ_SCALE_ABSMAX), (4, B.HQ_SCALE_STEP)])
@pytest.mark.parametrize("dt", [B.HQ_BF16, B.HQ_F16, B.HQ_F32])
def test_rotate_quantize_parity(rot, k, rows, cols, bits, mode, dt):
    banner("rq", rot, k, rows, cols, bits, mode, dt)
    rng = np.random.default_rng(rows * 31 + cols + k)
    V = rng.standard_normal((rows, cols))
    V[:, rng.choice(cols, max(1, cols // 100), replace=False)] *= 40.0   # outlier channels
    vb = WL.to_dtype_bits(V, dt)
    Vd = O.decode(vb, dt)
    step = None
    if mode == B.HQ_SCALE_STEP:
        step = float(np.float32(2.0 * np.sqrt(k if rot != B.HQ_ROT_BOTH else k * k) *
                                0.8 / np.sqrt(7.0)))
    both = rot == B.HQ_ROT_BOTH
    q = _rq(vb, dt, rows, cols, rot, k, bits, mode, step, codes=not both)
    ref_codes, ref_s = O.quantize_tensor(Vd, rot, k, bits, O.STEP if step else O.ABSMAX, step)
    got_t = q.codes_t_view().cpu().numpy()
    assert_codes(got_t.T, ref_codes, "codes_t")
    if not both:
        got = q.codes_view().cpu().numpy()
        np.testing.assert_array_equal(got_t, got.T)
        pad = q.codes.cpu().numpy()[:, cols:(cols + 15) // 16 * 16]
        assert not pad.any()
    assert_scale(float(q.scale.cpu()[0]), ref_s, "scale")
    # pitch padding is zero so whole 16-byte rows can be read by the GEMM
    pad_t = q.codes_t.cpu().numpy()[:, rows:(rows + 15) // 16 * 16]
    assert not pad_t.any()
    assert q.st.rows == rows and q.st.cols == cols and q.st.rot == rot and q.st.k == k


@pytest.mark.parametrize("k,rows,cols", [(256, 1024, 8448), (128, 2048, 4352)])
def test_rotate_quantize_both_pipelined(k, rows, cols):
    """X B and B X B with more items than workgroups (264 and 272 half tiles on 256): the
    next item's raw rows load into LDS during the current item's token-axis phase."""
    banner("rq-both-pipe", k, rows, cols)
    rng = np.random.default_rng(rows + cols + k)
    V = rng.standard_normal((rows, cols))
    V[:, rng.choice(cols, 8, replace=False)] *= 40.0
    vb = WL.to_dtype_bits(V, B.HQ_BF16)
    q = _rq(vb, B.HQ_BF16, rows, cols, B.HQ_ROT_BOTH, k, 8, B.HQ_SCALE_ABSMAX, codes=False)
    ref_codes, ref_s = O.quantize_tensor(O.decode(vb, B.HQ_BF16), B.HQ_ROT_BOTH, k, 8, O.ABSMAX)
    assert_codes(q.codes_t_view().cpu().numpy().T, ref_codes, "codes_t")
    assert_scale(float(q.scale.cpu()[0]), ref_s, "scale")


def _rq_both(vb, dt, rows, cols, k, bits, mode, fmt, step):
    q = T.QTensor(rows, cols, codes=False, codes_t=True)
    cfg = T.config(k, bits, mode, B.HQ_VARIANT_HQ, fmt)
    ws_bytes = B.hq_workspace_bytes(cfg, rows, cols, cols)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    src = T.device_tensor_from_bits(vb, dt, DEV)
    st = None if step is None else torch.tensor([step], dtype=torch.float32, device=DEV)
    B.check(B.hq_rotate_quantize(src.data_ptr(), dt, rows, cols, B.HQ_ROT_BOTH, cfg, T.ptr(st),
                                 q.st, ws.data_ptr(), ws_bytes, T.stream_ptr()), "rotate_quantize")
    torch.cuda.synchronize()
    return q.codes_t.cpu().numpy(), float(q.scale.cpu()[0])


@pytest.mark.parametrize("k", [16, 32, 64, 128])
@pytest.mark.parametrize("dt,bits,mode,fmt", [
    (B.HQ_BF16, 8, B.HQ_SCALE_ABSMAX, B.HQ_FMT_INT),
    (B.HQ_F16, 4, B.HQ_SCALE_STEP, B.HQ_FMT_INT),
    (B.HQ_BF16, 8, B.HQ_SCALE_ABSMAX, B.HQ_FMT_E4M3),
])
def test_both_narrow_items_match_half_tiles(k, dt, bits, mode, fmt, monkeypatch):
    """B X B with k <= 128 on 128 x 128 items (two workgroups per compute unit; 544 items on 512
    workgroups, so some take two) against the 256-row half-tile kernel, which HQ_BOTH_NARROW=0
    selects: the same rotation in the same order, so codes (every byte of the pitched buffer)
    and scale agree bit for bit; the integer codes are also compared with the oracle."""
    rows, cols = 2048, 4352
    banner("both-narrow", k, dt, bits, mode, fmt)
    rng = np.random.default_rng(900 + k)
    V = rng.standard_normal((rows, cols))
    V[:, rng.choice(cols, 8, replace=False)] *= 40.0
    vb = WL.to_dtype_bits(V, dt)
    step = float(np.float32(2.0 * k * 0.8 / np.sqrt(7.0))) if mode == B.HQ_SCALE_STEP else None
    narrow, s_n = _rq_both(vb, dt, rows, cols, k, bits, mode, fmt, step)
    monkeypatch.setenv("HQ_BOTH_NARROW", "0")
    halves, s_h = _rq_both(vb, dt, rows, cols, k, bits, mode, fmt, step)
    np.testing.assert_array_equal(narrow, halves)
    assert np.float32(s_n).tobytes() == np.float32(s_h).tobytes()
    if fmt == B.HQ_FMT_INT:
        ref_codes, ref_s = O.quantize_tensor(O.decode(vb, dt), B.HQ_ROT_BOTH, k, bits,
                                             O.STEP if step else O.ABSMAX, step)
        assert_codes(narrow[:, :rows].T, ref_codes, "codes_t")
        assert_scale(s_n, ref_s, "scale")


@pytest.mark.parametrize("k", [64, 128])
def test_layer_narrow_x_items(k, monkeypatch):
    """The HALO-2 forward's X pass on 128 x 128 items (X B row-major and B X B transposed codes
    from one pass pair), at a size with more items than workgroups: the whole layer against the
    oracle, and codes and outputs bit for bit against the 256-row half-tile kernel."""
    cfg = WL.config(5, N=2048, C=4352, D=256, k=k)
    banner("layer-narrow-x", k)
    inputs = WL.make_inputs(cfg)
    h = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    monkeypatch.setenv("HQ_BOTH_NARROW", "0")
    h0 = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    for key in h:
        np.testing.assert_array_equal(h[key], h0[key], err_msg=key)
    ora = run_oracle(cfg, inputs)
    compare_layer(cfg, h, ora, cfg["out_dtype"])


@pytest.mark.parametrize("cid,N,C,D", [(5, 1024, 2048, 768), (2, 512, 1024, 776), (3, 1000, 1024, 1000)])
def test_layer_output_store_hint(cid, N, C, D, monkeypatch):
    """The products store their outputs with the non-temporal hint (default) or without it
    (HQ_GEMM_NT=0): a cache hint only, so codes and outputs agree bit for bit (the
    2048 x 4096 x 4096-shaped case also takes the tile-pair exchange)."""
    cfg = WL.config(cid, N=N, C=C, D=D)
    banner("layer-store-hint", cid, N, C, D)
    inputs = WL.make_inputs(cfg)
    h = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    monkeypatch.setenv("HQ_GEMM_NT", "0")
    h0 = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    for key in h:
        np.testing.assert_array_equal(h[key], h0[key], err_msg=key)


@pytest.mark.parametrize("cid,N,C,D", [(5, 8192, 8192, 256), (5, 256, 8192, 8192),
                                     (5, 8192, 256, 8192)])
def test_layer_quant_order(cid, N, C, D, monkeypatch):
    """After an absmax pass over an input of 128 MiB or more (X, W and dY in turn) the quantize
    pass visits tiles last to first (default), or first to last with HQ_QUANT_REVERSE=0: each
    tile's codes depend only on the tile and the scale, so both orders give the same codes and
    outputs bit for bit."""
    cfg = WL.config(cid, N=N, C=C, D=D)
    banner("layer-quant-order", cid, N, C, D)
    inputs = WL.make_inputs(cfg)
    h = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    monkeypatch.setenv("HQ_QUANT_REVERSE", "0")
    h0 = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    for key in h:
        np.testing.assert_array_equal(h[key], h0[key], err_msg=key)


@pytest.mark.parametrize("cid,N,C,D", [(2, 512, 1024, 512), (4, 512, 1024, 768),
                                     (5, 1024, 2048, 512)])
def test_layer_prologue_valu_kernels(cid, N, C, D, monkeypatch):
    """HQ_PROLOGUE_VALU=1 runs every rotate-quantize pass of the layer on the VALU butterfly
    kernels instead of the matrix-core ones (whole tiles, k = 256 and 128): the layer still
    matches the oracle within the same bounds."""
    monkeypatch.setenv("HQ_PROLOGUE_VALU", "1")
    cfg = WL.config(cid, N=N, C=C, D=D)
    banner("layer-prologue-valu", cid, N, C, D)
    inputs = WL.make_inputs(cfg)
    h = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    ora = run_oracle(cfg, inputs)
    compare_layer(cfg, h, ora, cfg["out_dtype"])


@pytest.mark.parametrize("rot", [B.HQ_ROT_RIGHT, B.HQ_ROT_LEFT])
def test_rotate_quantize_single_layout(rot):
    """Only one code layout requested (the other is staged in the workspace)."""
    rng = np.random.default_rng(5)
    V = rng.standard_normal((256, 512))
    vb = WL.to_dtype_bits(V, B.HQ_BF16)
    ref, _ = O.quantize_tensor(O.decode(vb, B.HQ_BF16), rot, 32, 8)
    q1 = _rq(vb, B.HQ_BF16, 256, 512, rot, 32, 8, B.HQ_SCALE_ABSMAX, codes=True, codes_t=False)
    assert_codes(q1.codes_view().cpu().numpy(), ref, "rm only")
    q2 = _rq(vb, B.HQ_BF16, 256, 512, rot, 32, 8, B.HQ_SCALE_ABSMAX, codes=False, codes_t=True)
    assert_codes(q2.codes_t_view().cpu().numpy().T, ref, "t only")


def test_quantize_degenerate_tensors():
    """Zero tensor -> scale 0, codes 0; constant block -> energy in coefficient 0 only;
    a single outlier -> spread at equal magnitude over its block (codes +-127)."""
    rows, cols, k = 32, 256, 32
    Z = np.zeros((rows, cols))
    q = _rq(WL.to_dtype_bits(Z, B.HQ_BF16), B.HQ_BF16, rows, cols, B.HQ_ROT_RIGHT, k, 8,
            B.HQ_SCALE_ABSMAX)
    assert float(q.scale.cpu()[0]) == 0.0 and not q.codes_view().cpu().numpy().any()
    Cst = np.full((rows, cols), 0.5)
    q = _rq(WL.to_dtype_bits(Cst, B.HQ_BF16), B.HQ_BF16, rows, cols, B.HQ_ROT_RIGHT, k, 8,
            B.HQ_SCALE_ABSMAX)
    codes = q.codes_view().cpu().numpy()
    assert (codes[:, ::k] == 127).all()
    codes[:, ::k] = 0
    assert not codes.any()
    One = np.zeros((rows, cols))
    One[3, 40] = 2.0
    q = _rq(WL.to_dtype_bits(One, B.HQ_BF16), B.HQ_BF16, rows, cols, B.HQ_ROT_RIGHT, k, 8,
            B.HQ_SCALE_ABSMAX)
    codes = q.codes_view().cpu().numpy()
    assert (np.abs(codes[3, 32:64]) == 127).all()
    assert float(q.scale.cpu()[0]) == np.float32(2.0 / 127)


def test_quantize_empty_tensor():
    q = T.QTensor(0, 64)
    q.scale.fill_(5.0)
    cfg = T.config(32, 8, B.HQ_SCALE_ABSMAX, B.HQ_VARIANT_HQ)
    ws_bytes = B.hq_workspace_bytes(cfg, 1, 64, 64)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    x = torch.empty((1, 64), dtype=torch.bfloat16, device=DEV)
    B.check(B.hq_rotate_quantize(x.data_ptr(), B.HQ_BF16, 0, 64, B.HQ_ROT_RIGHT, cfg, None, q.st,
                                 ws.data_ptr(), ws_bytes, T.stream_ptr()), "empty")
    torch.cuda.synchronize()
    assert float(q.scale.cpu()[0]) == 0.0


# ------------------------------------------------------------- whole layer
REDUCED = {
    1: dict(),                                       # already small: 256 x 512 x 512
    2: dict(N=512, C=1024, D=768),
    3: dict(N=1000, C=1024, D=1000),                 # ragged token and output dims
    4: dict(N=512, C=768, D=1100),
    5: dict(N=256, C=1408, D=640),
}


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_layer_parity_reduced(cid):
    cfg = WL.config(cid, **REDUCED[cid])
    banner("layer", cfg["name"], cfg["N"], cfg["C"], cfg["D"])
    inputs = WL.make_inputs(cfg)
    res = run_gpu(cfg, inputs)
    h = host(res, cfg["out_dtype"])
    ora = run_oracle(cfg, inputs)
    stats = compare_layer(cfg, h, ora, cfg["out_dtype"])
    print("stats", stats, flush=True)
    # Same codes in, same products out: the GPU GEMM + epilogue against the oracle's products
    # evaluated on the GPU's own codes and scales.
    again = outputs_from_gpu_codes(cfg, h)
    for name, ref in again.items():
        err = rel_fro(h[name], rounded(ref, cfg["out_dtype"]))
        assert err <= 2e-3 * (1 if cfg["out_dtype"] != O.F32 else 1e-2), (name, err)


@pytest.mark.parametrize("cid", [2, 5])
def test_layer_parity_fp32_outputs(cid):
    """fp32 outputs: the GEMM + dequant + inverse rotation against the oracle's exact int64
    inverse rotation on the GPU's own codes, to 1e-5."""
    cfg = WL.config(cid, **REDUCED[cid])
    inputs = WL.make_inputs(cfg)
    res = run_gpu(cfg, inputs, out_dt=O.F32)
    h = host(res, O.F32)
    for name, ref in outputs_from_gpu_codes(cfg, h).items():
        err = rel_fro(h[name], ref)
        assert err <= 1e-5, (name, err)


@pytest.mark.parametrize("variant", [B.HQ_VARIANT_HALO0, B.HQ_VARIANT_HQ, B.HQ_VARIANT_HALO2])
@pytest.mark.parametrize("k", [1, 16, 64])
def test_layer_variants_and_k(variant, k):
    cfg = WL.config(2, N=256, C=320, D=192, k=k, variant=variant)
    if variant == B.HQ_VARIANT_HALO0:
        cfg["k"] = k
    inputs = WL.make_inputs(cfg)
    res = run_gpu(cfg, inputs)
    h = host(res, cfg["out_dtype"])
    ora = run_oracle(cfg, inputs)
    compare_layer(cfg, h, ora, cfg["out_dtype"])


@pytest.mark.parametrize("k,N,C,D", [(256, 256, 512, 1024), (256, 512, 1024, 776),
                                     (16, 256, 512, 1040), (128, 512, 768, 2048)])
def test_layer_narrow_dx(k, N, C, D):
    """HALO-2 dX with few 256 x 256 tiles runs on 256 x 128 tiles; with k = 256 the column
    rotation spans a pair of tiles, which exchange their rotated values and each finish half
    of the rows (k <= 128 rotates inside a tile). A ragged K puts a short last K step in every
    tile. Two layers in a row also check that the pair flags are cleared before each use."""
    for rep in range(2):
        cfg = WL.config(2, N=N, C=C, D=D, k=k)
        banner("narrow-dx", k, N, C, D, rep)
        inputs = WL.make_inputs(cfg)
        res = run_gpu(cfg, inputs, out_dt=O.F32)
        h = host(res, O.F32)
        for name, ref in outputs_from_gpu_codes(cfg, h).items():
            err = rel_fro(h[name], ref)
            assert err <= 1e-5, (name, err)


@pytest.mark.parametrize("N,C,D", [(256, 512, 1024), (512, 1024, 776)])
def test_layer_narrow_dx_fallback(N, C, D, monkeypatch):
    """The wait-free fallback of the tile pairs: with no polling, a tile that arrives before
    its partner publishes all its rows and leaves, and the partner finishes the whole block
    (or both finish their own rows when they meet). Forced from the host through the
    HQ_PAIR_SPIN hook; every kernel still ends normally."""
    monkeypatch.setenv("HQ_PAIR_SPIN", "0")
    for rep in range(2):
        cfg = WL.config(2, N=N, C=C, D=D, k=256)
        banner("narrow-dx-fallback", N, C, D, rep)
        inputs = WL.make_inputs(cfg)
        res = run_gpu(cfg, inputs, out_dt=O.F32)
        h = host(res, O.F32)
        for name, ref in outputs_from_gpu_codes(cfg, h).items():
            err = rel_fro(h[name], ref)
            assert err <= 1e-5, (name, err)


@pytest.mark.parametrize("spin", ["0", "40000"])
def test_layer_single_pass_x(spin, monkeypatch):
    """X under HALO-2 in one launch over a grid barrier (one half-tile item per workgroup).
    With no polling every workgroup but the last gives up, leaves its codes unwritten, and the
    quantize pass launched after it recomputes them from the published partials; with the
    default bound the single pass writes them. Forced from the host through HQ_SINGLE_SPIN;
    every kernel ends normally either way."""
    monkeypatch.setenv("HQ_SINGLE_SPIN", spin)
    for rep in range(2):
        cfg = WL.config(2, N=512, C=768, D=512)
        banner("single-pass-x", spin, rep)
        inputs = WL.make_inputs(cfg)
        res = run_gpu(cfg, inputs)
        h = host(res, cfg["out_dtype"])
        ora = run_oracle(cfg, inputs)
        compare_layer(cfg, h, ora, cfg["out_dtype"])


def test_layer_deterministic():
    cfg = WL.config(2, N=512, C=512, D=512)
    inputs = WL.make_inputs(cfg)
    a = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    b = host(run_gpu(cfg, inputs), cfg["out_dtype"])
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_layer_empty_tokens():
    """N = 0 tokens: nothing to compute, dW = 0 (no tokens to sum over)."""
    N, C, D = 0, 256, 128
    layer = T.Layer(N, C, D, 32, 8, B.HQ_SCALE_ABSMAX, B.HQ_VARIANT_HQ)
    x = torch.empty((N, C), dtype=torch.bfloat16, device=DEV)
    w = torch.randn((D, C), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    layer.fwd(x, w, y)
    dy = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((N, C), dtype=torch.bfloat16, device=DEV)
    layer.bwd_input(dy, dx)
    dw = torch.full((D, C), 7.0, dtype=torch.float32, device=DEV)
    layer.bwd_weight(dw)
    torch.cuda.synchronize()
    assert float(dw.abs().max()) == 0.0


# ------------------------------------------- grid-aligned inputs: exact end to end
def _blockdiag_h(n, k):
    return np.kron(np.eye(n // k, dtype=np.int64), O.hadamard(k).astype(np.int64))


def _ternary(rng, shape, density):
    """Entries in {-1, 0, 1}, nonzero with the given probability."""
    return rng.choice([-1, 0, 1], size=shape, p=[density / 2, 1 - density, density / 2])


def _run_exact_layer(cfg, xv, wv, gv, dt):
    """One layer step on exactly representable inputs (values given as float64), fp32 outputs."""
    inputs = {"x": WL.to_dtype_bits(xv, dt), "w": WL.to_dtype_bits(wv, dt),
              "dy": WL.to_dtype_bits(gv, dt)}
    for name, v in (("x", xv), ("w", wv), ("dy", gv)):
        np.testing.assert_array_equal(O.decode(inputs[name], dt), v)   # exact in the dtype
    cfg = dict(cfg, in_dtype=dt)
    res = run_gpu(cfg, inputs, out_dt=O.F32)
    return host(res, O.F32)


@pytest.mark.parametrize("k", [16, 128])
@pytest.mark.parametrize("dt", [B.HQ_BF16, B.HQ_F32])
def test_grid_aligned_hq_step_exact(k, dt):
    """HQ (right rotations, dY unrotated) on inputs built so that every rotated value is an
    integer and max |X B| = max |W B| = max |dY| = Qp: rotation -> absmax -> quantize must give
    those integers with s = 1 exactly (bit for bit), and since H H^T = k I, Y = X W^T,
    dX = dY W and dW = dY^T X exactly (INT4 page, §3.3). X and W are ternary, plus one k-block
    of 127/k per tensor, which rotates to 127 e_0; all sums stay far below 2^24, so the fp32
    sums of the kernels are exact. bf16 inputs take the matrix-core prologue, fp32 the VALU one."""
    banner("grid-aligned-hq", k, dt)
    rng = np.random.default_rng(900 + k + dt)
    N, C, D = 512, 512, 256
    X = _ternary(rng, (N, C), 0.3).astype(np.float64)
    W = _ternary(rng, (D, C), 0.3).astype(np.float64)
    G = rng.integers(-3, 4, size=(N, D)).astype(np.float64)
    X[0, :k] = 127.0 / k
    W[3, k:2 * k] = -127.0 / k
    G[5, 7] = 127.0
    Hc = _blockdiag_h(C, k)
    A, Bm = X @ Hc, W @ Hc                       # integer rotated values
    assert np.abs(A).max() == 127 and np.abs(Bm).max() == 127
    cfg = WL.config(2, N=N, C=C, D=D, k=k, variant=B.HQ_VARIANT_HQ)
    h = _run_exact_layer(cfg, X, W, G, dt)
    np.testing.assert_array_equal(h["qx"], A)
    np.testing.assert_array_equal(h["qw"], Bm)
    np.testing.assert_array_equal(h["qg"], G)
    assert h["sx"] == h["sw"] == h["sg"] == 1.0
    np.testing.assert_array_equal(h["y"], X @ W.T)
    np.testing.assert_array_equal(h["dx"], G @ W)
    np.testing.assert_array_equal(h["dw"], G.T @ X)


@pytest.mark.parametrize("k", [16, 64])
@pytest.mark.parametrize("dt", [B.HQ_BF16, B.HQ_F32])
def test_grid_aligned_halo2_backward_exact(k, dt):
    """HALO-2 backward on inputs whose rotated values are integers with max Qp: qG = Q(B_N dY),
    qXt = Q(B_N X B_C) and qW = Q(W B_C) are those integers with s = 1 (bit for bit), and the
    two backward products come out exactly: dX = B_N (qG qW) B_C / k^2 = dY W and
    dW = (qG^T qXt) B_C / k^2 = dY^T X (HALO page, Approach; INT4 page, §3.3). The forward
    output is checked against the oracle as usual."""
    banner("grid-aligned-halo2", k, dt)
    rng = np.random.default_rng(950 + k + dt)
    N, C, D = 512, 512, 256
    X = _ternary(rng, (N, C), min(0.2, 3.0 / k)).astype(np.float64)
    W = _ternary(rng, (D, C), 0.3).astype(np.float64)
    G = _ternary(rng, (N, D), 0.3).astype(np.float64)
    X[:k, :k] = 127.0 / (k * k)                  # B X B = 127 e_0 e_0^T on this block
    W[3, k:2 * k] = -127.0 / k
    G[k:2 * k, 9] = 127.0 / k                    # B G = 127 at row k, column 9
    Hn, Hc = _blockdiag_h(N, k), _blockdiag_h(C, k)
    Axt, Ag, Aw = Hn @ X @ Hc, Hn @ G, W @ Hc
    for a in (Axt, Ag, Aw):
        assert np.abs(a).max() == 127
    cfg = WL.config(2, N=N, C=C, D=D, k=k)
    h = _run_exact_layer(cfg, X, W, G, dt)
    np.testing.assert_array_equal(h["qxt_t"].T, Axt)
    np.testing.assert_array_equal(h["qg"], Ag)
    np.testing.assert_array_equal(h["qw"], Aw)
    assert h["sxt"] == h["sg"] == h["sw"] == 1.0
    np.testing.assert_array_equal(h["dx"], G @ W)
    np.testing.assert_array_equal(h["dw"], G.T @ X)
    ora = O.linear(X, W, G, k, 8, O.HALO2)
    assert_codes(h["qx"], ora["qx"], "qX")
    assert rel_fro(h["y"], ora["y"]) <= 1e-3
