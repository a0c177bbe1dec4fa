"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Codes and scales are compared in full (the oracle quantizes every tensor completely);
the dequantized outputs are compared on sampled entries the oracle computes one by one:
random rows x columns of Y, and k-aligned blocks of dX and dW (the inverse rotations only mix
within k-blocks, so an aligned block is self-contained). Outputs are compared against the
oracle's unrounded values: fp32 outputs within 1e-3, 16-bit outputs within 1e-3 plus the
dtype's unit roundoff (hq_testlib.out_bound).
"""
import numpy as np
import pytest

import oracle as O
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

from hq_testlib import assert_codes, assert_out, assert_scale, run_gpu

pytestmark = pytest.mark.gpu


def _dec(t, dt, rows=None, cols=None):
    """Decode a slice of a GPU output tensor to doubles."""
    if rows is not None:
        t = t[rows]
    if cols is not None:
        t = t[:, cols]
    return O.decode(T.bits_of(t.contiguous()), dt)


# Row blocks of dW that must be compared besides the random ones. At 8192 x 13824 x 5120 the
# weight-gradient product (computed as dW^T: 13824 x 5120 over 8192 tokens) runs as 256-wide
# tiles over dW rows [0, 4608) and a second launch of 128-wide tiles over [4608, 5120).
DW_ROWS = {5: [4608 - 64, 4608, 5120 - 64]}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_fullsize_sampled(cid):
    _check_sampled(WL.config(cid), 1000 + cid, dw_rows=DW_ROWS.get(cid, ()))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 4, 5])
def test_fullsize_fp32_outputs(cid):
    """The same launches with fp32 outputs: the dequantized-output bound (relative Frobenius
    error 1e-3) against the oracle's unrounded values, with no output rounding in between."""
    _check_sampled(WL.config(cid), 2000 + cid, dw_rows=DW_ROWS.get(cid, ()), out_dt=O.F32)


@pytest.mark.timeout(900)
def test_split_launch_with_column_rotation():
    """HALO-2 at k = 128 with 8192 tokens and C = 5120: the dX product (8192 x 5120, column
    rotation 128 wide) runs as 256-wide tiles over columns [0, 4096) and a second launch of
    128-wide tiles over [4096, 5120). Blocks on both sides of the seam and at the end are
    compared, besides the random samples."""
    _check_sampled(WL.config(5, N=8192, C=5120, D=256), 77,
                   dx_cols=[0, 4096 - 128, 4096, 5120 - 128])


def _check_sampled(cfg, seed, dx_cols=(), dw_rows=(), out_dt=None):
    N, C, D, k, v = cfg["N"], cfg["C"], cfg["D"], cfg["k"], cfg["variant"]
    out_dt = cfg["out_dtype"] if out_dt is None else out_dt
    print("[case] fullsize", cfg["name"], "out dtype", out_dt, flush=True)
    inputs = WL.make_inputs(cfg)
    res = run_gpu(cfg, inputs, out_dt=out_dt)
    L = res["layer"]
    print("[step] gpu done", flush=True)

    in_dt = cfg["in_dtype"]
    steps = inputs.get("steps") or {}
    mode = cfg["mode"]
    X = O.decode(inputs["x"], in_dt)
    qx, sx, qxt, sxt = O.quantize_x(X, k, cfg["bits"], v, mode, steps.get("x"), steps.get("xt"))
    del X
    assert_codes(L.qx.codes_view().cpu().numpy(), qx, "qX")
    assert_scale(float(L.qx.scale.cpu()[0]), sx, "sX")
    if L.qxt is not None:
        assert_codes(L.qxt.codes_t_view().cpu().numpy().T, qxt, "qXt")
        assert_scale(float(L.qxt.scale.cpu()[0]), sxt, "sXt")
    W = O.decode(inputs["w"], in_dt)
    qw, sw = O.quantize_w(W, k, cfg["bits"], v, mode, steps.get("w"))
    del W
    assert_codes(L.qw.codes_view().cpu().numpy(), qw, "qW")
    assert_scale(float(L.qw.scale.cpu()[0]), sw, "sW")
    print("[step] forward codes compared", flush=True)

    rng = np.random.default_rng(seed)
    rs = np.sort(rng.choice(N, min(N, 128), replace=False))
    cs = np.sort(rng.choice(D, min(D, 128), replace=False))
    y_ref = O.fwd_from_codes(qx, sx, qw, sw, k, v, rows=rs, cols=cs)
    assert_out(_dec(res["y"], out_dt, rows=rs, cols=cs), y_ref, out_dt, "Y sampled")

    if "dx" not in res:
        return
    G = O.decode(inputs["dy"], in_dt)
    qg, sg = O.quantize_g(G, k, cfg["bits"], v, mode, steps.get("g"))
    del G
    assert_codes(L.qg.codes_view().cpu().numpy(), qg, "qG")
    assert_scale(float(L.qg.scale.cpu()[0]), sg, "sG")
    print("[step] gradient codes compared", flush=True)

    kb = max(k, 16)
    blocks = [(int(rng.integers(0, N // kb)) * kb, int(rng.integers(0, C // kb)) * kb)
              for _ in range(2)]
    blocks += [(int(rng.integers(0, N // kb)) * kb, c) for c in dx_cols]
    for r0, c0 in blocks:
        ref = O.bwd_input_from_codes(qg, sg, qw, sw, k, v, row_block=(r0, kb), col_block=(c0, kb))
        assert_out(_dec(res["dx"][r0:r0 + kb, c0:c0 + kb], out_dt), ref, out_dt,
                   "dX block (%d, %d)" % (r0, c0))

    if "dw" not in res:
        return
    qxw = qxt if v == O.HALO2 else qx
    sxw = sxt if v == O.HALO2 else sx
    rows = [int(rng.integers(0, D - 64 + 1)) for _ in range(2)] + list(dw_rows)
    for r0 in rows:
        c0 = int(rng.integers(0, C // kb)) * kb
        ref = O.bwd_weight_from_codes(qg, sg, qxw, sxw, k, v, row_block=(r0, 64), col_block=(c0, kb))
        assert_out(_dec(res["dw"][r0:r0 + 64, c0:c0 + kb], out_dt), ref, out_dt,
                   "dW block (%d, %d)" % (r0, c0))


@pytest.mark.parametrize("rot", [1, 2])
def test_fwht_fullsize_sampled(rot):
    """hq_fwht at the size bench.py measures (8192 x 13824 bf16 -> bf16, k = 128, the X operand
    of the largest workload), on small-integer inputs so that every output is the exact
    rotation rounded once: sampled rows (RIGHT rotates within rows) or sampled k-row blocks on
    sampled column windows (LEFT mixes only within a block), bit for bit."""
    import torch
    from hadamard_rotated_precision_amd import binding as B
    rows, cols, k = 8192, 13824, 128
    print("[case] fwht fullsize rot", rot, flush=True)
    rng = np.random.default_rng(40 + rot)
    V = rng.integers(-8, 9, size=(rows, cols)).astype(np.float32)
    src = torch.from_numpy(V).to("cuda").to(torch.bfloat16)   # exact: |v| <= 8
    dst = torch.empty_like(src)
    B.check(B.hq_fwht(src.data_ptr(), B.HQ_BF16, dst.data_ptr(), B.HQ_BF16, rows, cols, rot, k,
                      T.stream_ptr()), "fwht")
    torch.cuda.synchronize()
    if rot == 1:
        for r in rng.choice(rows, 12, replace=False):
            got = T.bits_of(dst[int(r):int(r) + 1])
            ref = O.rotate(V[int(r):int(r) + 1].astype(np.float64), 1, k)
            np.testing.assert_array_equal(got, WL.to_dtype_bits(ref, WL.BF16))
    else:
        for b in rng.choice(rows // k, 6, replace=False):
            r0 = int(b) * k
            c0 = int(rng.integers(0, cols - 512))
            got = T.bits_of(dst[r0:r0 + k, c0:c0 + 512].contiguous())
            ref = O.rotate(V[r0:r0 + k, c0:c0 + 512].astype(np.float64), 2, k)
            np.testing.assert_array_equal(got, WL.to_dtype_bits(ref, WL.BF16))
