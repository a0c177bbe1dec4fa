"""GPU parity of the FP8 (E4M3) variant of the path against the oracle, through the C ABI.

The HALO summary page runs the three matmuls in FP8 as well as INT8 (Key results; an FP8 grid
stands in where FP6 hardware is missing, Limitations). Codes: at most one grid step apart on
at most 1e-4 of the entries (the GPU decides v * fp32(1/s), the oracle the exact quotient).
The FP8 products are exact, but the matrix cores sum them in fp32 in their own order, so the
GEMM is held to the floating-point output bound (relative Frobenius 1e-3 against the
oracle's exact sum) rather than bit-exactness; outputs as for INT8 (hq_testlib.out_bound).
"""
import numpy as np
import pytest
import torch

import oracle as O
from hadamard_rotated_precision_amd import binding as B
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

from hq_testlib import (compare_layer, fullsize_sampled, host, outputs_from_gpu_codes, rel_fro,
                        run_gpu, run_oracle, assert_out)

pytestmark = pytest.mark.gpu
DEV = "cuda"
E4M3_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def banner(*a):
    print("[case]", *a, flush=True)


def _padded(codes, K):
    """Rows padded to a multiple of 16 bytes with zero codes (the ABI's pitch rule)."""
    M = codes.shape[0]
    ld = (K + 15) // 16 * 16
    buf = np.zeros((M, ld), dtype=np.uint8)
    buf[:, :K] = codes
    return buf, ld


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (256, 256, 128), (300, 257, 1040),
                                   (513, 129, 4096), (64, 700, 48), (1024, 1536, 2048)])
def test_gemm_f8_f32_against_exact(M, N, K):
    banner("gemm-f8", M, N, K)
    rng = np.random.default_rng(M * 7 + N + K)
    # codes of a rotated, absmax-scaled tensor: mostly mid-range values, a few large ones
    A = rng.choice(E4M3_CODES, size=(M, K))
    Bt = rng.choice(E4M3_CODES, size=(N, K))
    a, lda = _padded(A, K)
    b, ldb = _padded(Bt, K)
    ad = torch.from_numpy(a).to(DEV)
    bd = torch.from_numpy(b).to(DEV)
    c = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    B.check(B.hq_gemm_f8_f32(ad.data_ptr(), lda, bd.data_ptr(), ldb, c.data_ptr(), M, N, K,
                             T.stream_ptr()), "hq_gemm_f8_f32")
    torch.cuda.synchronize()
    exact = O.gemm_f8(A, K, 1, Bt, 1, K, M, N, K).astype(np.float64) * 2.0 ** -18
    err = rel_fro(c.cpu().numpy(), exact)
    print("[gemm-f8] rel fro %.3g" % err, flush=True)
    assert err <= 1e-3


REDUCED = {
    2: dict(N=512, C=1024, D=768),
    4: dict(N=512, C=768, D=1100),
    5: dict(N=256, C=1408, D=640),
}


@pytest.mark.parametrize("cid", [2, 4, 5])
@pytest.mark.parametrize("out_dt", [None, O.F32])
def test_fp8_layer_parity_reduced(cid, out_dt):
    cfg = WL.config(cid, fmt=WL.E4M3, **REDUCED[cid])
    odt = cfg["out_dtype"] if out_dt is None else out_dt
    banner("fp8-layer", cfg["name"], cfg["N"], cfg["C"], cfg["D"], odt)
    inputs = WL.make_inputs(cfg)
    res = run_gpu(cfg, inputs, out_dt=odt)
    h = host(res, odt)
    ora = run_oracle(cfg, inputs)
    compare_layer(cfg, h, ora, odt)
    # same codes in: the FP8 GEMM + epilogue against the oracle's exact products on the GPU's
    # own codes and scales
    for name, ref in outputs_from_gpu_codes(cfg, h).items():
        assert_out(h[name], ref, odt, name + " (GPU codes)")


@pytest.mark.parametrize("k", [16, 64])
def test_fp8_grid_aligned_codes_exact(k):
    """X = A B_C / k with E4M3-representable A (entries in [1/8, 8] and one 448), given in
    fp32, which holds X exactly (bf16 would not: a sum of k such values needs more than 8
    significant bits). The FP8 forward quantizes X B_C back to A with s = 1 bit for bit, and
    Y equals X W^T up to the fp32 summation of the matrix cores."""
    banner("fp8-grid", k)
    rng = np.random.default_rng(60 + k)
    N, C, D = 512, 512, 256
    small = O.decode_e4m3(np.arange(0x20, 0x50, dtype=np.uint8))
    def draw(shape):
        v = rng.choice(small, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v[0, 0] = 448.0
        return v
    A, Bm = draw((N, C)), draw((D, C))
    H = np.kron(np.eye(C // k), O.hadamard(k).astype(np.float64))
    X, W = A @ H / k, Bm @ H / k
    cfg = dict(WL.config(2, N=N, C=C, D=D, k=k, variant=B.HQ_VARIANT_HQ, fmt=WL.E4M3),
               in_dtype=WL.F32, passes=("fwd",))
    inputs = {"x": WL.to_dtype_bits(X, WL.F32), "w": WL.to_dtype_bits(W, WL.F32), "dy": None}
    np.testing.assert_array_equal(O.decode(inputs["x"], WL.F32), X)
    res = run_gpu(cfg, inputs, out_dt=O.F32)
    h = host(res, O.F32)
    np.testing.assert_array_equal(O.decode_e4m3(h["qx"].view(np.uint8)), A)
    np.testing.assert_array_equal(O.decode_e4m3(h["qw"].view(np.uint8)), Bm)
    assert h["sx"] == h["sw"] == 1.0
    err = rel_fro(h["y"], X @ W.T)
    print("[fp8-grid] Y rel fro %.3g" % err, flush=True)
    assert err <= 1e-3


# dW rows on both sides of the head / tail launch seam at 8192 x 13824 x 5120 (dW computed as
# dW^T: 256-wide tiles over dW rows [0, 4608), 128-wide ones over [4608, 5120)), and the end
DW_SEAM = {5: (4608 - 64, 4608, 5120 - 64)}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 5])
def test_fp8_fullsize_sampled(cid):
    """The FP8 HALO-2 step at full size, 2048 x 4096 x 4096 (k = 256) and 8192 x 13824 x 5120
    (k = 128, the size bench.py times it at): codes and scales in full, outputs on sampled
    rows / k-aligned blocks against the oracle's exact values."""
    cfg = WL.config(cid, fmt=WL.E4M3)
    banner("fp8-fullsize", cfg["name"])
    fullsize_sampled(cfg, 3000 + cid, dw_rows=DW_SEAM.get(cid, ()))
