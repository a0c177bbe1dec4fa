"""C-ABI checks that need no GPU: the library loads, exports every symbol include/hq.h
declares, and rejects every invalid argument before any HIP call.

The pointers used here are fake addresses; every call below fails validation, which runs
before the first HIP call, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re

import pytest

from hadamard_rotated_precision_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000      # 16-byte aligned fake device address
FAKE_MIS = 0x10004  # misaligned


def declared_symbols():
    with open(os.path.join(ROOT, "include", "hq.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(hq_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = B.load()
    syms = declared_symbols()
    assert set(syms) == set(B.EXPORTS), syms
    for s in syms:
        assert hasattr(lib, s), s


def test_one_hip_runtime_in_process():
    """libhq binds to the HIP runtime torch loaded (the buffers and streams it gets are
    torch's), so the process maps exactly one libamdhip64."""
    B.load()
    maps = set()
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64" in path:
                maps.add(os.path.realpath(path))
    assert len(maps) == 1, maps


def test_version_status_pitch():
    assert B.hq_abi_version() == 2
    for code in range(12):
        assert isinstance(B.hq_status_string(code), str) and B.hq_status_string(code)
    assert B.hq_status_string(999) == "unknown status"
    assert B.hq_code_pitch(0) == 0 and B.hq_code_pitch(1) == 16 and B.hq_code_pitch(32) == 32
    assert B.hq_code_pitch(33) == 48


def cfg(k=32, bits=8, mode=B.HQ_SCALE_ABSMAX, variant=B.HQ_VARIANT_HALO2, fmt=B.HQ_FMT_INT):
    c = B.hq_config()
    c.k, c.bits, c.scale_mode, c.variant, c.format = k, bits, mode, variant, fmt
    return c


def qt(rows, cols, codes=FAKE, codes_t=FAKE, scale=FAKE, ld=None, ld_t=None, k=32, bits=8,
       rot=B.HQ_ROT_RIGHT):
    q = B.hq_qtensor()
    q.codes, q.codes_t, q.scale = codes, codes_t, scale
    q.rows, q.cols = rows, cols
    q.ld = B.hq_code_pitch(cols) if ld is None else ld
    q.ld_t = B.hq_code_pitch(rows) if ld_t is None else ld_t
    q.k, q.bits, q.rot = k, bits, rot
    return q


def test_workspace_bytes():
    # absmax partial arrays (4 x 1024 floats) plus a spare scalar, independent of the shapes
    small = B.hq_workspace_bytes(cfg(), 64, 64, 64)
    assert small >= 4 * 1024 * 4
    assert B.hq_workspace_bytes(cfg(), 8192, 13824, 5120) == small
    assert B.hq_workspace_bytes(cfg(k=3), 64, 64, 64) == 0
    assert B.hq_workspace_bytes(cfg(), -1, 64, 64) == 0


def rq(**kw):
    args = dict(src=FAKE, src_dtype=B.HQ_BF16, rows=64, cols=64, rot=B.HQ_ROT_RIGHT, cfg=cfg(),
                step=None, out=qt(64, 64), ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return B.hq_rotate_quantize(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(cfg=cfg(k=3)), "HQ_ERR_K"),
    (dict(cfg=cfg(k=512)), "HQ_ERR_K"),
    (dict(cfg=cfg(k=0)), "HQ_ERR_K"),
    (dict(cfg=cfg(bits=5)), "HQ_ERR_BITS"),
    (dict(cfg=cfg(bits=6)), "HQ_ERR_BITS"),                 # 6 bits only for FP6 codes
    (dict(cfg=cfg(bits=8, fmt=B.HQ_FMT_E2M3)), "HQ_ERR_BITS"),
    (dict(cfg=cfg(bits=4, fmt=B.HQ_FMT_E3M2)), "HQ_ERR_BITS"),
    (dict(cfg=cfg(bits=6, fmt=B.HQ_FMT_E4M3)), "HQ_ERR_BITS"),
    (dict(cfg=cfg(bits=6, fmt=4)), "HQ_ERR_MODE"),
    (dict(cfg=cfg(mode=7)), "HQ_ERR_MODE"),
    (dict(cfg=cfg(variant=3)), "HQ_ERR_MODE"),
    (dict(src_dtype=9), "HQ_ERR_DTYPE"),
    (dict(rot=4), "HQ_ERR_MODE"),
    (dict(rows=-1), "HQ_ERR_SHAPE"),
    (dict(cols=48), "HQ_ERR_SHAPE"),                       # 48 % 32 for a RIGHT rotation
    (dict(rot=B.HQ_ROT_LEFT, rows=40), "HQ_ERR_SHAPE"),    # token axis not divisible by k
    (dict(rot=B.HQ_ROT_BOTH, rows=40), "HQ_ERR_SHAPE"),
    (dict(cfg=cfg(mode=B.HQ_SCALE_STEP)), "HQ_ERR_NULL"),  # STEP without a step
    (dict(out=None), "HQ_ERR_NULL"),
    (dict(out=qt(64, 64, scale=None)), "HQ_ERR_NULL"),
    (dict(out=qt(64, 64, codes=None, codes_t=None)), "HQ_ERR_NULL"),
    (dict(src=None), "HQ_ERR_NULL"),
    (dict(out=qt(64, 64, codes=FAKE_MIS)), "HQ_ERR_ALIGN"),
    (dict(out=qt(64, 64, ld=72)), "HQ_ERR_ALIGN"),
    (dict(out=qt(64, 64, ld=48)), "HQ_ERR_SHAPE"),         # pitch shorter than cols
    (dict(out=qt(64, 64, codes_t=None), rot=B.HQ_ROT_BOTH), "HQ_ERR_NULL"),
    (dict(out=qt(64, 64), rot=B.HQ_ROT_BOTH), "HQ_ERR_MODE"),   # no row-major B V B codes
    (dict(ws=None), "HQ_ERR_WORKSPACE"),
    (dict(ws_bytes=100), "HQ_ERR_WORKSPACE"),
    (dict(ws=FAKE_MIS), "HQ_ERR_ALIGN"),
])
def test_rotate_quantize_validation(kw, expect):
    assert B.STATUS_NAMES[rq(**kw)] == expect


@pytest.mark.parametrize("fmt", [B.HQ_FMT_E2M3, B.HQ_FMT_E3M2])
def test_fp6_codes_pass_the_checks(fmt):
    """FP6 configurations pass every argument check and stop only at the device check."""
    assert B.STATUS_NAMES[rq(cfg=cfg(bits=6, fmt=fmt))] == "HQ_ERR_DEVICE"


@pytest.mark.parametrize("fmt", [B.HQ_FMT_E2M3, B.HQ_FMT_E3M2])
def test_fp6_statistics_are_refused(fmt):
    """The error sum and the Hadamard-size selection run on the integer and E4M3 grids only."""
    c = cfg(k=32, bits=6, fmt=fmt, variant=B.HQ_VARIANT_HQ)
    out = ctypes.c_double()
    r = B.hq_rotated_stat(FAKE, None, B.HQ_BF16, 64, 64, B.HQ_ROT_RIGHT, c, B.HQ_STAT_QERR, FAKE,
                          ctypes.addressof(out), FAKE, 1 << 30, None)
    assert B.STATUS_NAMES[r] == "HQ_ERR_MODE"
    carr = (ctypes.c_int32 * 1)(32)
    kb = ctypes.c_int32(0)
    r = B.hq_select_hadamard_k(FAKE, FAKE, B.HQ_BF16, 64, 64, 64, c, carr, 1, kb, None, FAKE,
                               1 << 30, None)
    assert B.STATUS_NAMES[r] == "HQ_ERR_MODE"


def fwd(**kw):
    N, C, D = kw.pop("N", 64), kw.pop("C", 64), kw.pop("D", 96)
    args = dict(x=FAKE, w=FAKE, in_dtype=B.HQ_BF16, N=N, C=C, D=D, cfg=cfg(), step_x=None,
                step_w=None, step_xt=None, y=FAKE, y_dtype=B.HQ_BF16, save_x=qt(N, C),
                save_xt=qt(N, C, rot=B.HQ_ROT_BOTH), save_w=qt(D, C), ws=FAKE,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return B.hq_linear_fwd(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(C=48), "HQ_ERR_SHAPE"),
    (dict(N=48), "HQ_ERR_SHAPE"),            # HALO2 needs N % k for the saved Q(B_N X B_C)
    (dict(y_dtype=5), "HQ_ERR_DTYPE"),
    (dict(save_x=None), "HQ_ERR_NULL"),
    (dict(save_w=qt(96, 64, codes=None)), "HQ_ERR_NULL"),
    (dict(save_xt=qt(64, 64, codes_t=None)), "HQ_ERR_NULL"),
    (dict(cfg=cfg(mode=B.HQ_SCALE_STEP), step_x=FAKE), "HQ_ERR_NULL"),
    (dict(y=None), "HQ_ERR_NULL"),
    (dict(ws_bytes=1024), "HQ_ERR_WORKSPACE"),
    (dict(save_w=qt(96, 64, ld_t=72)), "HQ_ERR_ALIGN"),
])
def test_linear_fwd_validation(kw, expect):
    assert B.STATUS_NAMES[fwd(**kw)] == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(C=48), "HQ_ERR_SHAPE"),
    (dict(y_dtype=5), "HQ_ERR_DTYPE"),
    (dict(save_x=None), "HQ_ERR_NULL"),
    (dict(cfg=cfg(k=12)), "HQ_ERR_K"),
    (dict(save_w=qt(96, 64, ld_t=72)), "HQ_ERR_ALIGN"),
])
def test_linear_fwd_noalloc_validation(kw, expect):
    """The no-allocation forward runs the same argument checks, before it looks up its
    scratch array or touches the device."""
    args = dict(x=FAKE, w=FAKE, in_dtype=B.HQ_BF16, N=64, C=64, D=96, cfg=cfg(), step_x=None,
                step_w=None, step_xt=None, y=FAKE, y_dtype=B.HQ_BF16, save_x=qt(64, 64),
                save_xt=qt(64, 64, rot=B.HQ_ROT_BOTH), save_w=qt(96, 64), stream=None)
    args.update(kw)
    assert B.STATUS_NAMES[B.hq_linear_fwd_noalloc(**args)] == expect


def test_linear_fwd_halo2_without_xt_is_allowed_before_device():
    # N = 48 is fine when the weight-gradient codes are not requested; the call then reaches
    # the device check, which fails on a machine without a gfx950 GPU.
    import torch
    if torch.cuda.is_available():
        pytest.skip("only meaningful without a GPU")
    assert B.STATUS_NAMES[fwd(N=48, save_xt=None, save_x=qt(48, 64),
                              ws_bytes=1 << 30)] == "HQ_ERR_DEVICE"


def bwd_in(**kw):
    N, C, D = 64, 64, 96
    args = dict(dy=FAKE, dy_dtype=B.HQ_BF16, N=N, C=C, D=D, cfg=cfg(), step_g=None,
                saved_w=qt(D, C), dx=FAKE, dx_dtype=B.HQ_BF16, save_g=qt(N, D, rot=B.HQ_ROT_LEFT),
                ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return B.hq_linear_bwd_input(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(saved_w=qt(96, 64, k=16)), "HQ_ERR_MISMATCH"),
    (dict(saved_w=qt(96, 64, bits=4)), "HQ_ERR_MISMATCH"),
    (dict(saved_w=qt(96, 64, rot=B.HQ_ROT_NONE)), "HQ_ERR_MISMATCH"),
    (dict(saved_w=qt(64, 64)), "HQ_ERR_MISMATCH"),
    (dict(saved_w=qt(96, 64, codes_t=None)), "HQ_ERR_NULL"),
    (dict(saved_w=None), "HQ_ERR_NULL"),
    (dict(save_g=None), "HQ_ERR_NULL"),
    (dict(cfg=cfg(mode=B.HQ_SCALE_STEP)), "HQ_ERR_NULL"),
    (dict(dx=None), "HQ_ERR_NULL"),
    (dict(dy_dtype=-1), "HQ_ERR_DTYPE"),
    (dict(ws=None), "HQ_ERR_WORKSPACE"),
])
def test_bwd_input_validation(kw, expect):
    assert B.STATUS_NAMES[bwd_in(**kw)] == expect


def bwd_w(**kw):
    N, C, D = 64, 64, 96
    args = dict(saved_g=qt(N, D, rot=B.HQ_ROT_LEFT), saved_x=qt(N, C, rot=B.HQ_ROT_BOTH), N=N,
                C=C, D=D, cfg=cfg(), dw=FAKE, dw_dtype=B.HQ_F32, ws=FAKE, ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return B.hq_linear_bwd_weight(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(saved_x=qt(64, 64, rot=B.HQ_ROT_RIGHT)), "HQ_ERR_MISMATCH"),  # HALO2 needs B_N X B_C
    (dict(saved_g=qt(64, 96, rot=B.HQ_ROT_NONE)), "HQ_ERR_MISMATCH"),
    (dict(cfg=cfg(variant=B.HQ_VARIANT_HQ)), "HQ_ERR_MISMATCH"),
    (dict(saved_g=qt(64, 96, rot=B.HQ_ROT_LEFT, ld_t=8)), "HQ_ERR_ALIGN"),
    (dict(dw=None), "HQ_ERR_NULL"),
    (dict(N=40), "HQ_ERR_SHAPE"),
])
def test_bwd_weight_validation(kw, expect):
    assert B.STATUS_NAMES[bwd_w(**kw)] == expect


def lss(**kw):
    N, C, D = 64, 64, 96
    args = dict(dy=FAKE, dy_dtype=B.HQ_BF16, saved_x=qt(N, C, bits=4, k=16), N=N, C=C, D=D,
                cfg=cfg(k=16, bits=4, variant=B.HQ_VARIANT_HQ), budget=32.0, uniforms=FAKE,
                dw=FAKE, dw_dtype=B.HQ_F32, probs=None, kept_idx=None, stats=None, ws=FAKE,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return B.hq_lss_bwd_weight(**args)


def test_lss_workspace_bytes():
    n = B.hq_lss_workspace_bytes(1000, 256, 512)
    assert n >= (256 + 512) * 1008 + 1000 * (4 + 8 + 8 + 1 + 4)
    assert B.hq_lss_workspace_bytes(-1, 8, 8) == 0
    assert B.hq_lss_workspace_bytes((1 << 21) + 1, 8, 8) == 0
    assert B.hq_lss_workspace_bytes(0, 8, 8) > 0


@pytest.mark.parametrize("kw,expect", [
    (dict(cfg=cfg(k=16, bits=8, variant=B.HQ_VARIANT_HQ)), "HQ_ERR_BITS"),
    (dict(cfg=cfg(k=16, bits=4, variant=B.HQ_VARIANT_HALO2)), "HQ_ERR_MODE"),
    (dict(cfg=cfg(k=3, bits=4, variant=B.HQ_VARIANT_HQ)), "HQ_ERR_K"),
    (dict(dy_dtype=5), "HQ_ERR_DTYPE"),
    (dict(dw_dtype=5), "HQ_ERR_DTYPE"),
    (dict(C=40), "HQ_ERR_SHAPE"),                                  # 40 % 16
    (dict(N=-1), "HQ_ERR_SHAPE"),
    (dict(N=(1 << 21) + 1), "HQ_ERR_SHAPE"),
    (dict(budget=float("nan")), "HQ_ERR_SHAPE"),
    (dict(budget=float("inf")), "HQ_ERR_SHAPE"),
    (dict(dy=None), "HQ_ERR_NULL"),
    (dict(uniforms=None), "HQ_ERR_NULL"),
    (dict(dw=None), "HQ_ERR_NULL"),
    (dict(saved_x=None), "HQ_ERR_NULL"),
    (dict(saved_x=qt(64, 64, bits=4, k=16, codes=None)), "HQ_ERR_NULL"),   # row-major codes
    (dict(saved_x=qt(64, 64, bits=4, k=16, scale=None)), "HQ_ERR_NULL"),
    (dict(saved_x=qt(64, 64, bits=8, k=16)), "HQ_ERR_MISMATCH"),
    (dict(saved_x=qt(64, 64, bits=4, k=32)), "HQ_ERR_MISMATCH"),
    (dict(saved_x=qt(64, 64, bits=4, k=16, rot=B.HQ_ROT_NONE)), "HQ_ERR_MISMATCH"),
    (dict(saved_x=qt(32, 64, bits=4, k=16)), "HQ_ERR_MISMATCH"),
    (dict(saved_x=qt(64, 64, bits=4, k=16, codes=FAKE_MIS)), "HQ_ERR_ALIGN"),
    (dict(saved_x=qt(64, 64, bits=4, k=16, ld=72)), "HQ_ERR_ALIGN"),
    (dict(saved_x=qt(64, 64, bits=4, k=16, ld=48)), "HQ_ERR_SHAPE"),
    (dict(probs=FAKE_MIS), "HQ_ERR_ALIGN"),
    (dict(ws=None), "HQ_ERR_WORKSPACE"),
    (dict(ws_bytes=1000), "HQ_ERR_WORKSPACE"),
    (dict(ws=FAKE_MIS), "HQ_ERR_ALIGN"),
])
def test_lss_validation(kw, expect):
    assert B.STATUS_NAMES[lss(**kw)] == expect


def test_lss_halo0_takes_unrotated_codes():
    # HALO0 samples against codes of X itself; with them the call reaches the device check,
    # which fails on a machine without a gfx950 GPU.
    import torch
    c = cfg(k=16, bits=4, variant=B.HQ_VARIANT_HALO0)
    assert B.STATUS_NAMES[lss(cfg=c)] == "HQ_ERR_MISMATCH"   # these codes carry B_C
    if torch.cuda.is_available():
        pytest.skip("only meaningful without a GPU")
    assert B.STATUS_NAMES[lss(cfg=c, C=40, saved_x=qt(64, 40, bits=4, k=16,
                                                      rot=B.HQ_ROT_NONE))] == "HQ_ERR_DEVICE"


@pytest.mark.parametrize("kw,expect", [
    (dict(k=6), "HQ_ERR_K"),
    (dict(rot=B.HQ_ROT_BOTH), "HQ_ERR_MODE"),
    (dict(cols=40), "HQ_ERR_SHAPE"),
    (dict(src=None), "HQ_ERR_NULL"),
    (dict(dst_dtype=3), "HQ_ERR_DTYPE"),
])
def test_fwht_validation(kw, expect):
    args = dict(src=FAKE, src_dtype=B.HQ_F32, dst=FAKE, dst_dtype=B.HQ_F32, rows=32, cols=64,
                rot=B.HQ_ROT_RIGHT, k=32, stream=None)
    args.update(kw)
    assert B.STATUS_NAMES[B.hq_fwht(**args)] == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(path=3), "HQ_ERR_MODE"),
    (dict(path=B.HQ_FWHT_MATRIX), "HQ_ERR_MODE"),                       # fp32: no matrix path
    (dict(path=B.HQ_FWHT_MATRIX, src_dtype=B.HQ_BF16, dst_dtype=B.HQ_BF16, rows=64,
          cols=512, k=8), "HQ_ERR_MODE"),                              # k < 16
    (dict(path=B.HQ_FWHT_MATRIX, src_dtype=B.HQ_BF16, dst_dtype=B.HQ_BF16, rows=64,
          cols=500, k=4), "HQ_ERR_MODE"),                              # partial tile
    (dict(path=B.HQ_FWHT_MATRIX, src_dtype=B.HQ_BF16, dst_dtype=B.HQ_BF16, rows=64,
          cols=512, k=32, src=FAKE + 2), "HQ_ERR_MODE"),               # unaligned
    (dict(path=B.HQ_FWHT_BUTTERFLY, k=6), "HQ_ERR_K"),
])
def test_fwht_path_validation(kw, expect):
    args = dict(src=FAKE, src_dtype=B.HQ_F32, dst=FAKE, dst_dtype=B.HQ_F32, rows=32, cols=64,
                rot=B.HQ_ROT_RIGHT, k=32, path=B.HQ_FWHT_AUTO, stream=None)
    args.update(kw)
    assert B.STATUS_NAMES[B.hq_fwht_path(**args)] == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(lda=8), "HQ_ERR_SHAPE"),
    (dict(lda=72, K=64), "HQ_ERR_ALIGN"),
    (dict(a=FAKE_MIS), "HQ_ERR_ALIGN"),
    (dict(c=None), "HQ_ERR_NULL"),
    (dict(M=-1), "HQ_ERR_SHAPE"),
])
def test_gemm_validation(kw, expect):
    args = dict(a=FAKE, lda=64, b_t=FAKE, ldb=64, c=FAKE, M=32, N=32, K=64, stream=None)
    args.update(kw)
    assert B.STATUS_NAMES[B.hq_gemm_i8_i32(**args)] == expect


def test_empty_calls_return_ok_without_device():
    # zero-size products have nothing to launch
    assert B.hq_gemm_i8_i32(None, 16, None, 16, None, 0, 0, 0, None) == B.HQ_OK
    assert B.hq_fwht(None, B.HQ_F32, None, B.HQ_F32, 0, 64, B.HQ_ROT_RIGHT, 32, None) == B.HQ_OK


def test_no_compute_symbol_outside_header():
    """Every exported hq_* function is declared in the header (no hidden entry points)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(m for m in re.findall(r"\bT (hq_[a-z0-9_]+)\b", out)))
    assert exported == declared_symbols()
