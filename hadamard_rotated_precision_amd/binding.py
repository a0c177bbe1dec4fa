"""Thin ctypes binding of libhq (include/hq.h): the same entry-point names, argument
marshalling only. Every step of the computation runs in the HIP kernels behind the C ABI;
torch is used by the helpers below only to allocate device memory and to name streams.

Loading fails loudly when the library is missing and cannot be built: there is no fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# HQ_LIB_PATH names another build of the same sources (the host-sanitizer test's); there is
# still no fallback when the named library is missing
LIB_PATH = os.environ.get("HQ_LIB_PATH") or os.path.join(HERE, "libhq.so")

# enums of include/hq.h
HQ_OK = 0
STATUS_NAMES = {0: "HQ_OK", 1: "HQ_ERR_NULL", 2: "HQ_ERR_SHAPE", 3: "HQ_ERR_K", 4: "HQ_ERR_BITS",
                5: "HQ_ERR_DTYPE", 6: "HQ_ERR_MODE", 7: "HQ_ERR_WORKSPACE", 8: "HQ_ERR_MISMATCH",
                9: "HQ_ERR_DEVICE", 10: "HQ_ERR_LAUNCH", 11: "HQ_ERR_ALIGN"}
HQ_F32, HQ_F16, HQ_BF16 = 0, 1, 2
HQ_ROT_NONE, HQ_ROT_RIGHT, HQ_ROT_LEFT, HQ_ROT_BOTH = 0, 1, 2, 3
HQ_SCALE_ABSMAX, HQ_SCALE_STEP = 0, 1
HQ_VARIANT_HALO0, HQ_VARIANT_HQ, HQ_VARIANT_HALO2 = 0, 1, 2
HQ_FWHT_AUTO, HQ_FWHT_BUTTERFLY, HQ_FWHT_MATRIX = 0, 1, 2
HQ_FMT_INT, HQ_FMT_E4M3, HQ_FMT_E2M3, HQ_FMT_E3M2 = 0, 1, 2, 3

EXPORTS = ["hq_abi_version", "hq_status_string", "hq_code_pitch", "hq_workspace_bytes",
           "hq_rotate_quantize", "hq_linear_fwd", "hq_linear_fwd_noalloc", "hq_linear_bwd_input",
           "hq_linear_bwd_weight", "hq_fwht", "hq_fwht_path", "hq_gemm_i8_i32", "hq_gemm_f8_f32",
           "hq_profile_start", "hq_profile_stop", "hq_profile_records",
           "hq_bmm_workspace_bytes", "hq_bmm_fwd", "hq_bmm_bwd_input", "hq_bmm_bwd_weight",
           "hq_rotated_stat", "hq_cold_start_step", "hq_select_hadamard_k",
           "hq_lss_workspace_bytes", "hq_lss_bwd_weight"]
HQ_STAT_ABS_SUM, HQ_STAT_QERR, HQ_STAT_LSQ_GRAD = 0, 1, 2
HQ_MAX_K_CANDIDATES = 16
HQ_KIND_GEMM, HQ_KIND_ROT_ABSMAX, HQ_KIND_ROT_QUANT, HQ_KIND_ROT_STORE = 0, 1, 2, 3
HQ_KIND_TRANSPOSE, HQ_KIND_MISC, HQ_KIND_COUNT = 4, 5, 6
KIND_NAMES = ["gemm", "rot_absmax", "rot_quant", "rot_store", "transpose", "misc"]


class hq_config(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("format", ctypes.c_int32)]


class hq_qtensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("codes_t", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("ld_t", ctypes.c_int64), ("k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("rot", ctypes.c_int32), ("format", ctypes.c_int32)]


class hq_lss_stats(ctypes.Structure):
    _fields_ = [("kept", ctypes.c_int32), ("s8", ctypes.c_float), ("s_hi", ctypes.c_float),
                ("s_lo", ctypes.c_float)]


class hq_profile_stat(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("count", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("units", ctypes.c_double)]


class hq_profile_record(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("ms", ctypes.c_double), ("units", ctypes.c_double)]


class HQError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS_NAMES.get(status, status),
                                          hq_status_string(status)))


_lib = None


def load(build_if_missing=True):
    """Load libhq.so; build it first only when no built library exists."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError("libhq.so is not built (run hadamard_rotated_precision_amd/build.py)")
        from . import build as _build
        _build.build()
    # The device buffers and streams handed to libhq come from torch's HIP runtime. torch
    # ships its own libamdhip64 (same soname as the system one); loading torch first makes
    # libhq bind to that copy, so the process holds one HIP runtime, not two that do not
    # share allocations.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    lib.hq_abi_version.restype = i32
    lib.hq_abi_version.argtypes = []
    lib.hq_status_string.restype = ctypes.c_char_p
    lib.hq_status_string.argtypes = [i32]
    lib.hq_code_pitch.restype = i64
    lib.hq_code_pitch.argtypes = [i64]
    lib.hq_workspace_bytes.restype = sz
    lib.hq_workspace_bytes.argtypes = [P(hq_config), i64, i64, i64]
    lib.hq_rotate_quantize.restype = i32
    lib.hq_rotate_quantize.argtypes = [vp, i32, i64, i64, i32, P(hq_config), vp, P(hq_qtensor),
                                       vp, sz, vp]
    lib.hq_linear_fwd.restype = i32
    lib.hq_linear_fwd.argtypes = [vp, vp, i32, i64, i64, i64, P(hq_config), vp, vp, vp, vp, i32,
                                  P(hq_qtensor), P(hq_qtensor), P(hq_qtensor), vp, sz, vp]
    lib.hq_linear_fwd_noalloc.restype = i32
    lib.hq_linear_fwd_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, P(hq_config), vp, vp, vp,
                                          vp, i32, P(hq_qtensor), P(hq_qtensor), P(hq_qtensor), vp]
    lib.hq_linear_bwd_input.restype = i32
    lib.hq_linear_bwd_input.argtypes = [vp, i32, i64, i64, i64, P(hq_config), vp, P(hq_qtensor),
                                        vp, i32, P(hq_qtensor), vp, sz, vp]
    lib.hq_linear_bwd_weight.restype = i32
    lib.hq_linear_bwd_weight.argtypes = [P(hq_qtensor), P(hq_qtensor), i64, i64, i64,
                                         P(hq_config), vp, i32, vp, sz, vp]
    lib.hq_fwht.restype = i32
    lib.hq_fwht.argtypes = [vp, i32, vp, i32, i64, i64, i32, i32, vp]
    lib.hq_bmm_workspace_bytes.restype = sz
    lib.hq_bmm_workspace_bytes.argtypes = [P(hq_config)]
    lib.hq_bmm_fwd.restype = i32
    lib.hq_bmm_fwd.argtypes = [vp, vp, i32, i64, i64, i64, i64, P(hq_config), vp, vp, vp, vp, i32,
                               P(hq_qtensor), P(hq_qtensor), P(hq_qtensor), vp, sz, vp]
    lib.hq_bmm_bwd_input.restype = i32
    lib.hq_bmm_bwd_input.argtypes = [vp, i32, i64, i64, i64, i64, P(hq_config), vp, P(hq_qtensor),
                                     vp, i32, P(hq_qtensor), vp, sz, vp]
    lib.hq_bmm_bwd_weight.restype = i32
    lib.hq_bmm_bwd_weight.argtypes = [P(hq_qtensor), P(hq_qtensor), i64, i64, i64, i64,
                                      P(hq_config), vp, i32, vp, sz, vp]
    lib.hq_rotated_stat.restype = i32
    lib.hq_rotated_stat.argtypes = [vp, vp, i32, i64, i64, i32, P(hq_config), i32, vp, vp, vp,
                                    sz, vp]
    lib.hq_cold_start_step.restype = i32
    lib.hq_cold_start_step.argtypes = [vp, i32, i64, i64, i32, P(hq_config), vp, vp, sz, vp]
    lib.hq_select_hadamard_k.restype = i32
    lib.hq_select_hadamard_k.argtypes = [vp, vp, i32, i64, i64, i64, P(hq_config), vp, i32, vp,
                                         vp, vp, sz, vp]
    lib.hq_lss_workspace_bytes.restype = sz
    lib.hq_lss_workspace_bytes.argtypes = [i64, i64, i64]
    lib.hq_lss_bwd_weight.restype = i32
    lib.hq_lss_bwd_weight.argtypes = [vp, i32, P(hq_qtensor), i64, i64, i64, P(hq_config),
                                      ctypes.c_double, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.hq_gemm_f8_f32.restype = i32
    lib.hq_gemm_f8_f32.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, vp]
    lib.hq_fwht_path.restype = i32
    lib.hq_fwht_path.argtypes = [vp, i32, vp, i32, i64, i64, i32, i32, i32, vp]
    lib.hq_gemm_i8_i32.restype = i32
    lib.hq_gemm_i8_i32.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, vp]
    lib.hq_profile_start.restype = i32
    lib.hq_profile_start.argtypes = [ctypes.c_uint32]
    lib.hq_profile_stop.restype = i32
    lib.hq_profile_stop.argtypes = [P(hq_profile_stat), i32]
    lib.hq_profile_records.restype = i32
    lib.hq_profile_records.argtypes = [P(hq_profile_record), i32]
    _lib = lib
    return lib


def _ref(s):
    return None if s is None else ctypes.byref(s)


# ------------------------------------------------ entry points, same names as the C ABI
def hq_abi_version():
    return load().hq_abi_version()


def hq_status_string(status):
    return load().hq_status_string(status).decode()


def hq_code_pitch(cols):
    return load().hq_code_pitch(cols)


def hq_workspace_bytes(cfg, N, C, D):
    return load().hq_workspace_bytes(ctypes.byref(cfg), N, C, D)


def hq_rotate_quantize(src, src_dtype, rows, cols, rot, cfg, step, out, ws, ws_bytes, stream):
    return load().hq_rotate_quantize(src, src_dtype, rows, cols, rot, _ref(cfg), step, _ref(out),
                                     ws, ws_bytes, stream)


def hq_linear_fwd(x, w, in_dtype, N, C, D, cfg, step_x, step_w, step_xt, y, y_dtype, save_x,
                  save_xt, save_w, ws, ws_bytes, stream):
    return load().hq_linear_fwd(x, w, in_dtype, N, C, D, _ref(cfg), step_x, step_w, step_xt, y,
                                y_dtype, _ref(save_x), _ref(save_xt), _ref(save_w), ws,
                                ws_bytes, stream)


def hq_linear_fwd_noalloc(x, w, in_dtype, N, C, D, cfg, step_x, step_w, step_xt, y, y_dtype,
                          save_x, save_xt, save_w, stream):
    return load().hq_linear_fwd_noalloc(x, w, in_dtype, N, C, D, _ref(cfg), step_x, step_w,
                                        step_xt, y, y_dtype, _ref(save_x), _ref(save_xt),
                                        _ref(save_w), stream)


def hq_linear_bwd_input(dy, dy_dtype, N, C, D, cfg, step_g, saved_w, dx, dx_dtype, save_g, ws,
                        ws_bytes, stream):
    return load().hq_linear_bwd_input(dy, dy_dtype, N, C, D, _ref(cfg), step_g, _ref(saved_w),
                                      dx, dx_dtype, _ref(save_g), ws, ws_bytes, stream)


def hq_linear_bwd_weight(saved_g, saved_x, N, C, D, cfg, dw, dw_dtype, ws, ws_bytes, stream):
    return load().hq_linear_bwd_weight(_ref(saved_g), _ref(saved_x), N, C, D, _ref(cfg), dw,
                                       dw_dtype, ws, ws_bytes, stream)


def hq_fwht(src, src_dtype, dst, dst_dtype, rows, cols, rot, k, stream):
    return load().hq_fwht(src, src_dtype, dst, dst_dtype, rows, cols, rot, k, stream)


def hq_fwht_path(src, src_dtype, dst, dst_dtype, rows, cols, rot, k, path, stream):
    return load().hq_fwht_path(src, src_dtype, dst, dst_dtype, rows, cols, rot, k, path, stream)


def hq_gemm_i8_i32(a, lda, b_t, ldb, c, M, N, K, stream):
    return load().hq_gemm_i8_i32(a, lda, b_t, ldb, c, M, N, K, stream)


def hq_bmm_workspace_bytes(cfg):
    return load().hq_bmm_workspace_bytes(ctypes.byref(cfg))


def hq_bmm_fwd(x, w, in_dtype, batch, N, C, D, cfg, step_x, step_w, step_xt, y, y_dtype, save_x,
               save_xt, save_w, ws, ws_bytes, stream):
    return load().hq_bmm_fwd(x, w, in_dtype, batch, N, C, D, _ref(cfg), step_x, step_w, step_xt,
                             y, y_dtype, _ref(save_x), _ref(save_xt), _ref(save_w), ws, ws_bytes,
                             stream)


def hq_bmm_bwd_input(dy, dy_dtype, batch, N, C, D, cfg, step_g, saved_w, dx, dx_dtype, save_g, ws,
                     ws_bytes, stream):
    return load().hq_bmm_bwd_input(dy, dy_dtype, batch, N, C, D, _ref(cfg), step_g,
                                   _ref(saved_w), dx, dx_dtype, _ref(save_g), ws, ws_bytes, stream)


def hq_bmm_bwd_weight(saved_g, saved_x, batch, N, C, D, cfg, dw, dw_dtype, ws, ws_bytes, stream):
    return load().hq_bmm_bwd_weight(_ref(saved_g), _ref(saved_x), batch, N, C, D, _ref(cfg), dw,
                                    dw_dtype, ws, ws_bytes, stream)


def hq_rotated_stat(src, grad, dtype, rows, cols, rot, cfg, stat, scale, out, ws, ws_bytes,
                    stream):
    return load().hq_rotated_stat(src, grad, dtype, rows, cols, rot, _ref(cfg), stat, scale, out,
                                  ws, ws_bytes, stream)


def hq_cold_start_step(src, dtype, rows, cols, rot, cfg, step, ws, ws_bytes, stream):
    return load().hq_cold_start_step(src, dtype, rows, cols, rot, _ref(cfg), step, ws, ws_bytes,
                                     stream)


def hq_select_hadamard_k(x, w, dtype, N, C, D, cfg, candidates, n_candidates, k_best, errors, ws,
                         ws_bytes, stream):
    """candidates: a ctypes int32 array; k_best: a ctypes int32; errors: a ctypes double array
    of 2 * n_candidates, or None (host memory)."""
    return load().hq_select_hadamard_k(x, w, dtype, N, C, D, _ref(cfg), candidates, n_candidates,
                                       ctypes.byref(k_best),
                                       None if errors is None else errors, ws, ws_bytes, stream)


def hq_lss_workspace_bytes(N, C, D):
    return load().hq_lss_workspace_bytes(N, C, D)


def hq_lss_bwd_weight(dy, dy_dtype, saved_x, N, C, D, cfg, budget, uniforms, dw, dw_dtype, probs,
                      kept_idx, stats, ws, ws_bytes, stream):
    """probs, kept_idx, stats: device pointers (stats: one hq_lss_stats on the device) or None."""
    return load().hq_lss_bwd_weight(dy, dy_dtype, _ref(saved_x), N, C, D, _ref(cfg), budget,
                                    uniforms, dw, dw_dtype, probs, kept_idx, stats, ws, ws_bytes,
                                    stream)


def hq_gemm_f8_f32(a, lda, b_t, ldb, c, M, N, K, stream):
    return load().hq_gemm_f8_f32(a, lda, b_t, ldb, c, M, N, K, stream)


def hq_profile_start(kind_mask):
    return load().hq_profile_start(kind_mask)


def hq_profile_stop(stats, n_stats):
    return load().hq_profile_stop(stats, n_stats)


def hq_profile_records(out, cap):
    return load().hq_profile_records(out, cap)


def profile_records():
    """The per-launch records of the last hq_profile_stop: a list of (kind name, ms, units)."""
    n = hq_profile_records(None, 0)
    arr = (hq_profile_record * max(n, 1))()
    n = hq_profile_records(arr, n)
    return [(KIND_NAMES[arr[i].kind], arr[i].ms, arr[i].units) for i in range(n)]


def profile_stop_dict():
    """hq_profile_stop into a {kind name: (count, total_ms, units)} dict."""
    arr = (hq_profile_stat * HQ_KIND_COUNT)()
    check(hq_profile_stop(arr, HQ_KIND_COUNT), "hq_profile_stop")
    return {KIND_NAMES[i]: (arr[i].count, arr[i].total_ms, arr[i].units)
            for i in range(HQ_KIND_COUNT)}


def check(status, where=""):
    if status != HQ_OK:
        raise HQError(status, where)
    return status
