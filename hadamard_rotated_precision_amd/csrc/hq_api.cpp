// hq_api.cpp — the C ABI of libhq (declared in include/hq.h): argument validation, workspace
// layout and the order of kernel passes for each entry point. Every argument check runs
// before the first HIP call, so invalid calls launch nothing (and need no GPU).
#include "../../include/hq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string.h>

#include "hq_internal.hpp"

namespace {

using hq::ColPass;
using hq::GemmPass;
using hq::RowPass;

constexpr size_t kPartialBytes = 4 * hq::kMaxPartials * sizeof(float);   // 4 partial arrays
constexpr size_t kAlign = 256;
constexpr size_t kBarBytes = hq::kBarWordsInts * sizeof(int32_t);          // grid-barrier words

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t pitch16(int64_t n) { return (n + 15) / 16 * 16; }
bool is_pow2_k(int32_t k) { return k >= 1 && k <= 256 && (k & (k - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dt(int32_t dt) { return dt == HQ_F32 || dt == HQ_F16 || dt == HQ_BF16; }
int qmax(int32_t bits) { return bits == 4 ? 7 : 127; }

hq_status check_cfg(const hq_config* cfg) {
  if (!cfg) return HQ_ERR_NULL;
  if (!is_pow2_k(cfg->k)) return HQ_ERR_K;
  if (cfg->bits != 4 && cfg->bits != 8) return HQ_ERR_BITS;
  if (cfg->scale_mode != HQ_SCALE_ABSMAX && cfg->scale_mode != HQ_SCALE_STEP) return HQ_ERR_MODE;
  if (cfg->variant < HQ_VARIANT_HALO0 || cfg->variant > HQ_VARIANT_HALO2) return HQ_ERR_MODE;
  return HQ_OK;
}

// Workspace: the absmax partial arrays, one spare device float, the grid-barrier words of the
// single-pass two-sided kernel, then (when the dX product of a HALO-2 layer runs on paired
// 256 x 128 tiles) the pair flags and published tiles.
size_t ws_need() { return kPartialBytes + kAlign + kBarBytes; }

int64_t dx_split_tiles(const hq_config* cfg, int64_t N, int64_t C, int64_t D) {
  if (cfg->variant != HQ_VARIANT_HALO2 || cfg->k <= 1) return 0;
  return hq::gemm_split_tiles(N, C, D, hq::EPI_SCALE, cfg->k, cfg->k, false);
}

size_t ws_need_layer(const hq_config* cfg, int64_t N, int64_t C, int64_t D) {
  const int64_t split = dx_split_tiles(cfg, N, C, D);
  return ws_need() + (split > 0 ? hq::gemm_split_bytes(split) : 0);
}

hq_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return HQ_OK;
  if (!ws || ws_bytes < need) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  return HQ_OK;
}

struct Ws {
  float* part[4];
  float* spare;
  int32_t* bar;  // grid-barrier words (kBarWordsInts)
  void* split;   // tile-pair area (only as large as the call's hq_workspace_bytes allows)
  explicit Ws(void* base) {
    char* b = static_cast<char*>(base);
    for (int i = 0; i < 4; ++i) part[i] = reinterpret_cast<float*>(b + i * hq::kMaxPartials * 4);
    spare = reinterpret_cast<float*>(b + kPartialBytes);
    bar = reinterpret_cast<int32_t*>(b + kPartialBytes + kAlign);
    split = b + ws_need();
  }
};

// Properties of the device current at the first call, read once.
struct DeviceInfo {
  hq_status st = HQ_ERR_DEVICE;
  int cus = 0;   // compute units visible to this process
};

const DeviceInfo& device_info() {
  static std::once_flag once;
  static DeviceInfo info;
  std::call_once(once, [] {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    if (strncmp(prop.gcnArchName, "gfx950", 6) == 0) info.st = HQ_OK;
    info.cus = prop.multiProcessorCount;
  });
  return info;
}

hq_status device_ok() { return device_info().st; }

#define HQ_TRY(expr)                                  \
  do {                                                \
    if ((expr) != hipSuccess) return HQ_ERR_LAUNCH;   \
  } while (0)

// Rotate -> scale -> quantize one tensor into row-major and/or transposed codes (one absmax
// pass unless a step is given, then one quantize pass that writes both layouts).
hq_status quantize_tensor(const void* src, int32_t dt, int64_t rows, int64_t cols, int32_t rot,
                          int32_t k, int32_t bits, const float* step, int8_t* codes, int64_t ld,
                          int8_t* codes_t, int64_t ld_t, float* scale, const Ws& ws,
                          int part_slot, hipStream_t st, int32_t* zero_ptr = nullptr,
                          int64_t zero_n = 0) {
  if (rows * cols == 0) {   // empty tensor: scale = step (or 0); there are no codes to write
    HQ_TRY(hq::write_scale(scale, step, st));
    return HQ_OK;
  }
  if (k == 1) rot = HQ_ROT_NONE;
  hq::ProPass p;
  p.src = src;
  p.in_dt = dt;
  p.rows = rows;
  p.cols = cols;
  p.qp = qmax(bits);
  p.partials = ws.part[part_slot];
  p.step = step;
  p.zero_ptr = zero_ptr;
  p.zero_n = zero_n;
  if (rot == HQ_ROT_BOTH) {
    // the two-sided kernel also produces the right-only scale: park it in the workspace
    p.kind = hq::PRO_BOTH;
    p.k = k;
    p.step2 = step;
    p.scale_out = ws.spare;
    p.scale_out2 = scale;
    p.codes_t = codes_t;
    p.ld_t = ld_t;
    if (codes) return HQ_ERR_MODE;   // row-major codes of B V B are not produced
  } else {
    p.kind = (rot == HQ_ROT_LEFT) ? hq::PRO_LEFT : hq::PRO_RIGHT;
    p.k = (rot == HQ_ROT_NONE) ? 1 : k;
    p.scale_out = scale;
    p.codes = codes;
    p.ld = ld;
    p.codes_t = codes_t;
    p.ld_t = ld_t;
  }
  if (!step) {
    p.nparts = hq::pro_grid(p);
    HQ_TRY(hq::pro_pass(p, hq::OP_ABSMAX, st));
  }
  HQ_TRY(hq::pro_pass(p, hq::OP_QUANT, st));
  return HQ_OK;
}

// The two-sided pass of X under HALO-2: Q(X B) row-major and Q(B X B) transposed.
hq::ProPass x_both_pass(const void* src, int32_t dt, int64_t rows, int64_t cols, int32_t k,
                        int32_t bits, const float* step_x, const float* step_xt, hq_qtensor* qx,
                        hq_qtensor* qxt, const Ws& ws) {
  hq::ProPass p;
  p.kind = hq::PRO_BOTH;
  p.src = src;
  p.in_dt = dt;
  p.rows = rows;
  p.cols = cols;
  p.k = k;
  p.qp = qmax(bits);
  p.partials = ws.part[0];
  p.step = step_x;
  p.step2 = step_xt;
  p.scale_out = qx->scale;
  p.scale_out2 = qxt->scale;
  p.codes = qx->codes;
  p.ld = qx->ld;
  p.codes_t = qxt->codes_t;
  p.ld_t = qxt->ld_t;
  return p;
}

// X under HALO-2: one pass pair writes Q(X B) row-major and Q(B X B) transposed.
hq_status quantize_x_both(const void* src, int32_t dt, int64_t rows, int64_t cols, int32_t k,
                          int32_t bits, const float* step_x, const float* step_xt,
                          hq_qtensor* qx, hq_qtensor* qxt, const Ws& ws, hipStream_t st) {
  if (rows * cols == 0) {
    HQ_TRY(hq::write_scale(qx->scale, step_x, st));
    HQ_TRY(hq::write_scale(qxt->scale, step_xt, st));
    return HQ_OK;
  }
  hq::ProPass p = x_both_pass(src, dt, rows, cols, k, bits, step_x, step_xt, qx, qxt, ws);
  if (!step_x) {
    p.nparts = hq::pro_grid(p);
    HQ_TRY(hq::pro_pass(p, hq::OP_ABSMAX, st));
  }
  HQ_TRY(hq::pro_pass(p, hq::OP_QUANT, st));
  return HQ_OK;
}

// Output qtensor: a scale is always needed; code buffers only for a non-empty tensor.
hq_status check_qt_out(const hq_qtensor* q, bool need_codes, bool need_any, int64_t elems) {
  if (!q || !q->scale) return HQ_ERR_NULL;
  if (elems == 0) return HQ_OK;
  if (need_codes && !q->codes) return HQ_ERR_NULL;
  if (need_any && !q->codes && !q->codes_t) return HQ_ERR_NULL;
  return HQ_OK;
}

hq_status check_pitches(const hq_qtensor* q, int64_t rows, int64_t cols) {
  if (q->codes) {
    if (!aligned16(q->codes) || q->ld % 16 != 0) return HQ_ERR_ALIGN;
    if (q->ld < cols) return HQ_ERR_SHAPE;
  }
  if (q->codes_t) {
    if (!aligned16(q->codes_t) || q->ld_t % 16 != 0) return HQ_ERR_ALIGN;
    if (q->ld_t < rows) return HQ_ERR_SHAPE;
  }
  return HQ_OK;
}

void fill_meta(hq_qtensor* q, int64_t rows, int64_t cols, int32_t k, int32_t bits, int32_t rot) {
  q->rows = rows;
  q->cols = cols;
  q->k = k;
  q->bits = bits;
  q->rot = rot;
}

hq_status check_saved(const hq_qtensor* q, int64_t rows, int64_t cols, const hq_config* cfg,
                      int32_t rot) {
  if (!q || !q->scale || (!q->codes_t && rows * cols > 0)) return HQ_ERR_NULL;
  if (q->rows != rows || q->cols != cols || q->k != cfg->k || q->bits != cfg->bits ||
      q->rot != rot)
    return HQ_ERR_MISMATCH;
  if (!aligned16(q->codes_t) || q->ld_t % 16 != 0) return HQ_ERR_ALIGN;
  if (q->ld_t < rows) return HQ_ERR_SHAPE;
  return HQ_OK;
}

int32_t x_rot(int32_t variant) { return variant == HQ_VARIANT_HALO0 ? HQ_ROT_NONE : HQ_ROT_RIGHT; }
int32_t g_rot(int32_t variant) { return variant == HQ_VARIANT_HALO2 ? HQ_ROT_LEFT : HQ_ROT_NONE; }
int32_t xt_rot(int32_t variant) {
  return variant == HQ_VARIANT_HALO2 ? HQ_ROT_BOTH : x_rot(variant);
}

#define HQ_CHECK(expr)             \
  do {                             \
    hq_status s_ = (expr);         \
    if (s_ != HQ_OK) return s_;    \
  } while (0)

}  // namespace

extern "C" {

int32_t hq_abi_version(void) { return HQ_ABI_VERSION; }

const char* hq_status_string(int32_t s) {
  switch (s) {
    case HQ_OK: return "ok";
    case HQ_ERR_NULL: return "a required pointer is NULL";
    case HQ_ERR_SHAPE: return "bad shape (negative, not divisible by k, or mismatched pitch)";
    case HQ_ERR_K: return "k must be a power of two in [1, 256]";
    case HQ_ERR_BITS: return "bits must be 4 or 8";
    case HQ_ERR_DTYPE: return "unsupported dtype";
    case HQ_ERR_MODE: return "bad rotation, scale mode or variant";
    case HQ_ERR_WORKSPACE: return "workspace missing or too small";
    case HQ_ERR_MISMATCH: return "saved quantized tensor does not match this call";
    case HQ_ERR_DEVICE: return "no usable gfx950 device";
    case HQ_ERR_LAUNCH: return "kernel launch failed";
    case HQ_ERR_ALIGN: return "device pointer or code pitch not 16-byte aligned";
  }
  return "unknown status";
}

int64_t hq_code_pitch(int64_t cols) { return cols < 0 ? 0 : pitch16(cols); }

size_t hq_workspace_bytes(const hq_config* cfg, int64_t N, int64_t C, int64_t D) {
  if (check_cfg(cfg) != HQ_OK || N < 0 || C < 0 || D < 0) return 0;
  return ws_need_layer(cfg, N, C, D);
}

hq_status hq_rotate_quantize(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                             int32_t rot, const hq_config* cfg, const float* step,
                             hq_qtensor* out, void* ws, size_t ws_bytes, void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(src_dtype)) return HQ_ERR_DTYPE;
  if (rot < HQ_ROT_NONE || rot > HQ_ROT_BOTH) return HQ_ERR_MODE;
  if (rows < 0 || cols < 0) return HQ_ERR_SHAPE;
  if ((rot == HQ_ROT_RIGHT || rot == HQ_ROT_BOTH) && cols % cfg->k) return HQ_ERR_SHAPE;
  if ((rot == HQ_ROT_LEFT || rot == HQ_ROT_BOTH) && rows % cfg->k) return HQ_ERR_SHAPE;
  if (cfg->scale_mode == HQ_SCALE_STEP && !step) return HQ_ERR_NULL;
  HQ_CHECK(check_qt_out(out, false, true, rows * cols));
  if (rows * cols > 0 && !src) return HQ_ERR_NULL;
  HQ_CHECK(check_pitches(out, rows, cols));
  if (rot == HQ_ROT_BOTH && !out->codes_t && rows * cols > 0) return HQ_ERR_NULL;
  if (rot == HQ_ROT_BOTH && out->codes && cfg->k > 1) return HQ_ERR_MODE;
  HQ_CHECK(check_ws(ws, ws_bytes, ws_need()));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws w(ws);
  HQ_CHECK(quantize_tensor(src, src_dtype, rows, cols, rot, cfg->k, cfg->bits,
                           cfg->scale_mode == HQ_SCALE_STEP ? step : nullptr, out->codes,
                           out->ld, out->codes_t, out->ld_t, out->scale, w, 0, st));
  fill_meta(out, rows, cols, cfg->k, cfg->bits, rot);
  return HQ_OK;
}

hq_status hq_linear_fwd(const void* x, const void* w, int32_t in_dtype, int64_t N, int64_t C,
                        int64_t D, const hq_config* cfg, const float* step_x,
                        const float* step_w, const float* step_xt, void* y, int32_t y_dtype,
                        hq_qtensor* save_x, hq_qtensor* save_xt, hq_qtensor* save_w, void* ws,
                        size_t ws_bytes, void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(in_dtype) || !valid_dt(y_dtype)) return HQ_ERR_DTYPE;
  if (N < 0 || C < 0 || D < 0) return HQ_ERR_SHAPE;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HALO0 && C % k) return HQ_ERR_SHAPE;
  const bool want_xt = (v == HQ_VARIANT_HALO2) && save_xt != nullptr;
  if (want_xt && N % k) return HQ_ERR_SHAPE;
  const bool stepm = cfg->scale_mode == HQ_SCALE_STEP;
  if (stepm && (!step_x || !step_w || (want_xt && !step_xt))) return HQ_ERR_NULL;
  if ((N * C > 0 && !x) || (D * C > 0 && !w) || (N * D > 0 && !y)) return HQ_ERR_NULL;
  HQ_CHECK(check_qt_out(save_x, true, true, N * C));
  HQ_CHECK(check_qt_out(save_w, true, true, D * C));
  HQ_CHECK(check_pitches(save_x, N, C));
  HQ_CHECK(check_pitches(save_w, D, C));
  if (want_xt) {
    if (!save_xt->scale || (!save_xt->codes_t && N * C > 0)) return HQ_ERR_NULL;
    HQ_CHECK(check_pitches(save_xt, N, C));
  }
  HQ_CHECK(check_ws(ws, ws_bytes, hq_workspace_bytes(cfg, N, C, D)));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws wsp(ws);
  const int32_t rx = x_rot(v);
  const bool two_sided = want_xt && !save_x->codes_t && !save_xt->codes && k > 1;
  // X's two-sided pass runs in a single launch over a grid barrier when it is small enough;
  // W's quantize pass, launched just before, zeroes the barrier words
  hq::ProPass px;
  bool single = false;
  if (two_sided && !stepm && N * C > 0) {
    px = x_both_pass(x, in_dtype, N, C, k, cfg->bits, nullptr, nullptr, save_x, save_xt, wsp);
    single = hq::pro_single_ok(px, device_info().cus) && D * C > 0;
  }
  HQ_CHECK(quantize_tensor(w, in_dtype, D, C, rx, k, cfg->bits, stepm ? step_w : nullptr,
                           save_w->codes, save_w->ld, save_w->codes_t, save_w->ld_t,
                           save_w->scale, wsp, 2, st, single ? wsp.bar : nullptr,
                           single ? hq::kBarWordsInts : 0));
  fill_meta(save_w, D, C, k, cfg->bits, rx);
  if (single) {
    px.nparts = hq::pro_grid(px);
    HQ_TRY(hq::pro_single_pass(px, wsp.bar, st));
    HQ_TRY(hq::pro_fixup_pass(px, wsp.bar, st));
  } else if (two_sided) {
    HQ_CHECK(quantize_x_both(x, in_dtype, N, C, k, cfg->bits, stepm ? step_x : nullptr,
                             stepm ? step_xt : nullptr, save_x, save_xt, wsp, st));
  } else {
    HQ_CHECK(quantize_tensor(x, in_dtype, N, C, rx, k, cfg->bits, stepm ? step_x : nullptr,
                             save_x->codes, save_x->ld, save_x->codes_t, save_x->ld_t,
                             save_x->scale, wsp, 0, st));
    if (want_xt)
      HQ_CHECK(quantize_tensor(x, in_dtype, N, C, HQ_ROT_BOTH, k, cfg->bits,
                               stepm ? step_xt : nullptr, k > 1 ? nullptr : save_xt->codes,
                               save_xt->ld, save_xt->codes_t, save_xt->ld_t, save_xt->scale,
                               wsp, 1, st));
  }
  fill_meta(save_x, N, C, k, cfg->bits, rx);
  if (want_xt) fill_meta(save_xt, N, C, k, cfg->bits, HQ_ROT_BOTH);
  GemmPass g;
  g.cus = device_info().cus;
  g.a = save_x->codes;
  g.lda = save_x->ld;
  g.b = save_w->codes;
  g.ldb = save_w->ld;
  g.M = N;
  g.N = D;
  g.K = C;
  g.epi = hq::EPI_SCALE;
  g.c = y;
  g.ldc = D;
  g.out_dt = y_dtype;
  g.sa = save_x->scale;
  g.sb = save_w->scale;
  g.kmul = (v == HQ_VARIANT_HALO0) ? 1.0f : 1.0f / static_cast<float>(k);
  HQ_TRY(hq::gemm_pass(g, st));
  return HQ_OK;
}

hq_status hq_linear_bwd_input(const void* dy, int32_t dy_dtype, int64_t N, int64_t C, int64_t D,
                              const hq_config* cfg, const float* step_g,
                              const hq_qtensor* saved_w, void* dx, int32_t dx_dtype,
                              hq_qtensor* save_g, void* ws, size_t ws_bytes, void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(dy_dtype) || !valid_dt(dx_dtype)) return HQ_ERR_DTYPE;
  if (N < 0 || C < 0 || D < 0) return HQ_ERR_SHAPE;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HALO0 && C % k) return HQ_ERR_SHAPE;
  if (v == HQ_VARIANT_HALO2 && N % k) return HQ_ERR_SHAPE;
  const bool stepm = cfg->scale_mode == HQ_SCALE_STEP;
  if (stepm && !step_g) return HQ_ERR_NULL;
  if ((N * D > 0 && !dy) || (N * C > 0 && !dx)) return HQ_ERR_NULL;
  HQ_CHECK(check_saved(saved_w, D, C, cfg, x_rot(v)));
  HQ_CHECK(check_qt_out(save_g, true, true, N * D));
  HQ_CHECK(check_pitches(save_g, N, D));
  HQ_CHECK(check_ws(ws, ws_bytes, hq_workspace_bytes(cfg, N, C, D)));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws wsp(ws);
  const int32_t rg = g_rot(v);
  // paired dX tiles need their arrival flags at zero: the quantize pass clears them
  const int64_t split = dx_split_tiles(cfg, N, C, D);
  HQ_CHECK(quantize_tensor(dy, dy_dtype, N, D, rg, k, cfg->bits, stepm ? step_g : nullptr,
                           save_g->codes, save_g->ld, save_g->codes_t, save_g->ld_t,
                           save_g->scale, wsp, 0, st,
                           split > 0 ? static_cast<int32_t*>(wsp.split) : nullptr, split));
  fill_meta(save_g, N, D, k, cfg->bits, rg);
  // dX = [B_N] (qG qW) [B_C] sG sW / k^e, dequantized and inverse-rotated in the GEMM epilogue.
  GemmPass g;
  g.cus = device_info().cus;
  g.epi = hq::EPI_SCALE;
  g.sa = save_g->scale;
  g.sb = saved_w->scale;
  g.c = dx;
  g.out_dt = dx_dtype;
  g.ldc = C;
  g.K = D;
  if (v == HQ_VARIANT_HQ) {
    // only the columns (C) rotate: compute dX^T = qW^T qG^T so C is the tile's row axis,
    // where the epilogue rotates in registers, and store it transposed
    g.a = saved_w->codes_t;
    g.lda = saved_w->ld_t;
    g.b = save_g->codes;
    g.ldb = save_g->ld;
    g.M = C;
    g.N = N;
    g.km = k;
    g.trans_out = true;
    g.kmul = 1.0f / static_cast<float>(k);
  } else {
    g.a = save_g->codes;
    g.lda = save_g->ld;
    g.b = saved_w->codes_t;
    g.ldb = saved_w->ld_t;
    g.M = N;
    g.N = C;
    if (v == HQ_VARIANT_HALO2) {   // rows (tokens) and columns (C) both rotate
      g.km = k;
      g.kn = k;
      g.kmul = 1.0f / static_cast<float>(k * k);
      if (split > 0) {
        g.split_ws = wsp.split;
        g.split_cnt_zeroed = N * D > 0;   // the quantize pass above ran and cleared them
      }
    }
  }
  HQ_TRY(hq::gemm_pass(g, st));
  return HQ_OK;
}

hq_status hq_linear_bwd_weight(const hq_qtensor* saved_g, const hq_qtensor* saved_x, int64_t N,
                               int64_t C, int64_t D, const hq_config* cfg, void* dw,
                               int32_t dw_dtype, void* ws, size_t ws_bytes, void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(dw_dtype)) return HQ_ERR_DTYPE;
  if (N < 0 || C < 0 || D < 0) return HQ_ERR_SHAPE;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HALO0 && C % k) return HQ_ERR_SHAPE;
  if (v == HQ_VARIANT_HALO2 && N % k) return HQ_ERR_SHAPE;
  if (D * C > 0 && !dw) return HQ_ERR_NULL;
  HQ_CHECK(check_saved(saved_g, N, D, cfg, g_rot(v)));
  HQ_CHECK(check_saved(saved_x, N, C, cfg, xt_rot(v)));
  HQ_CHECK(check_ws(ws, ws_bytes, hq_workspace_bytes(cfg, N, C, D)));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws wsp(ws);
  // dW = (qG^T qX') [B_C] sG sX' / k^e. When C rotates, compute dW^T = qX'^T qG so C is the
  // tile's row axis (rotated in registers) and store it transposed.
  GemmPass g;
  g.cus = device_info().cus;
  g.epi = hq::EPI_SCALE;
  g.sa = saved_g->scale;
  g.sb = saved_x->scale;
  g.c = dw;
  g.out_dt = dw_dtype;
  g.ldc = C;
  g.K = N;
  if (v == HQ_VARIANT_HALO0) {
    g.a = saved_g->codes_t;
    g.lda = saved_g->ld_t;
    g.b = saved_x->codes_t;
    g.ldb = saved_x->ld_t;
    g.M = D;
    g.N = C;
  } else {
    g.a = saved_x->codes_t;
    g.lda = saved_x->ld_t;
    g.b = saved_g->codes_t;
    g.ldb = saved_g->ld_t;
    g.M = C;
    g.N = D;
    g.km = k;
    g.trans_out = true;
    g.kmul = (v == HQ_VARIANT_HALO2) ? 1.0f / static_cast<float>(k * k) : 1.0f / static_cast<float>(k);
  }
  HQ_TRY(hq::gemm_pass(g, st));
  return HQ_OK;
}

hq_status hq_fwht(const void* src, int32_t src_dtype, void* dst, int32_t dst_dtype, int64_t rows,
                  int64_t cols, int32_t rot, int32_t k, void* stream) {
  if (!valid_dt(src_dtype) || !valid_dt(dst_dtype)) return HQ_ERR_DTYPE;
  if (!is_pow2_k(k)) return HQ_ERR_K;
  if (rot != HQ_ROT_NONE && rot != HQ_ROT_RIGHT && rot != HQ_ROT_LEFT) return HQ_ERR_MODE;
  if (rows < 0 || cols < 0) return HQ_ERR_SHAPE;
  if (rot == HQ_ROT_RIGHT && cols % k) return HQ_ERR_SHAPE;
  if (rot == HQ_ROT_LEFT && rows % k) return HQ_ERR_SHAPE;
  if (rows * cols > 0 && (!src || !dst)) return HQ_ERR_NULL;
  if (rows * cols == 0) return HQ_OK;
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rot == HQ_ROT_LEFT && k > 1 &&
      hq::fwht_left_mma_ok(src, src_dtype, dst, dst_dtype, rows, cols, k)) {
    HQ_TRY(hq::fwht_left_mma(src, src_dtype, rows, cols, k, dst, st));
    return HQ_OK;
  }
  if (rot == HQ_ROT_LEFT && k > 1) {
    ColPass c;
    c.src = src;
    c.in_dt = src_dtype;
    c.rows = rows;
    c.cols = cols;
    c.k = k;
    c.dst = dst;
    c.out_dt = dst_dtype;
    HQ_TRY(hq::cols_pass(c, st));
    return HQ_OK;
  }
  if (rot == HQ_ROT_RIGHT && k > 1 &&
      hq::fwht_right_mma_ok(src, src_dtype, dst, dst_dtype, rows, cols, k)) {
    HQ_TRY(hq::fwht_right_mma(src, src_dtype, rows, cols, k, dst, st));
    return HQ_OK;
  }
  RowPass r;
  r.src = src;
  r.in_dt = src_dtype;
  r.rows = rows;
  r.cols = cols;
  r.k = (rot == HQ_ROT_RIGHT) ? k : 1;
  r.dst = dst;
  r.out_dt = dst_dtype;
  HQ_TRY(hq::rows_pass(r, st));
  return HQ_OK;
}

hq_status hq_gemm_i8_i32(const int8_t* a, int64_t lda, const int8_t* b_t, int64_t ldb,
                         int32_t* c, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K < 0) return HQ_ERR_SHAPE;
  if ((M * K > 0 && !a) || (N * K > 0 && !b_t) || (M * N > 0 && !c)) return HQ_ERR_NULL;
  if (lda < K || ldb < K) return HQ_ERR_SHAPE;
  if (lda % 16 || ldb % 16 || (a && !aligned16(a)) || (b_t && !aligned16(b_t))) return HQ_ERR_ALIGN;
  if (M * N == 0) return HQ_OK;
  HQ_CHECK(device_ok());
  GemmPass g;
  g.cus = device_info().cus;
  g.a = a;
  g.lda = lda;
  g.b = b_t;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi = hq::EPI_I32;
  g.c = c;
  g.ldc = N;
  HQ_TRY(hq::gemm_pass(g, static_cast<hipStream_t>(stream)));
  return HQ_OK;
}

}  // extern "C"
