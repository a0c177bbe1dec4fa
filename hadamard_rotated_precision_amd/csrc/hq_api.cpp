// hq_api.cpp — the C ABI of libhq (declared in include/hq.h): argument validation, workspace
// layout and the order of kernel passes for each entry point. Every argument check runs
// before the first HIP call, so invalid calls launch nothing (and need no GPU).
#include "../../include/hq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
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
// Float-format codes (E4M3, or the FP6 formats kept as E4M3 bytes): the FP8 product serves them.
bool is_f8(const hq_config* cfg) { return cfg->format != HQ_FMT_INT; }
bool is_fp6(const hq_config* cfg) {
  return cfg->format == HQ_FMT_E2M3 || cfg->format == HQ_FMT_E3M2;
}
// integer grid bound Qp (float formats: 448, only where an integer is needed)
int qmax(const hq_config* cfg) { return is_f8(cfg) ? 448 : (cfg->bits == 4 ? 7 : 127); }
// the scale's divisor: Qp, or the format's largest value (E4M3 448, E2M3 7.5, E3M2 28)
float qmax_f(const hq_config* cfg) {
  switch (cfg->format) {
    case HQ_FMT_E4M3: return 448.0f;
    case HQ_FMT_E2M3: return 7.5f;
    case HQ_FMT_E3M2: return 28.0f;
  }
  return static_cast<float>(qmax(cfg));
}
// the prologue's float grid: 0 E4M3, 1 E2M3, 2 E3M2
int fgrid(const hq_config* cfg) {
  return cfg->format == HQ_FMT_E2M3 ? 1 : (cfg->format == HQ_FMT_E3M2 ? 2 : 0);
}

hq_status check_cfg(const hq_config* cfg) {
  if (!cfg) return HQ_ERR_NULL;
  if (!is_pow2_k(cfg->k)) return HQ_ERR_K;
  if (cfg->format != HQ_FMT_INT && cfg->format != HQ_FMT_E4M3 && !is_fp6(cfg)) return HQ_ERR_MODE;
  if (cfg->format == HQ_FMT_INT && cfg->bits != 4 && cfg->bits != 8) return HQ_ERR_BITS;
  if (cfg->format == HQ_FMT_E4M3 && cfg->bits != 8) return HQ_ERR_BITS;
  if (is_fp6(cfg) && cfg->bits != 6) return HQ_ERR_BITS;
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
                          int32_t k, const hq_config* cfg, const float* step, int8_t* codes, int64_t ld,
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
  p.qp = qmax(cfg);
  p.f8 = is_f8(cfg);
  p.qmaxf = qmax_f(cfg);
  p.fgrid = fgrid(cfg);
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
                        const hq_config* cfg, const float* step_x, const float* step_xt,
                        hq_qtensor* qx, hq_qtensor* qxt, const Ws& ws) {
  hq::ProPass p;
  p.kind = hq::PRO_BOTH;
  p.src = src;
  p.in_dt = dt;
  p.rows = rows;
  p.cols = cols;
  p.k = k;
  p.qp = qmax(cfg);
  p.f8 = is_f8(cfg);
  p.qmaxf = qmax_f(cfg);
  p.fgrid = fgrid(cfg);
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
                          const hq_config* cfg, const float* step_x, const float* step_xt,
                          hq_qtensor* qx, hq_qtensor* qxt, const Ws& ws, hipStream_t st) {
  if (rows * cols == 0) {
    HQ_TRY(hq::write_scale(qx->scale, step_x, st));
    HQ_TRY(hq::write_scale(qxt->scale, step_xt, st));
    return HQ_OK;
  }
  hq::ProPass p = x_both_pass(src, dt, rows, cols, k, cfg, step_x, step_xt, qx, qxt, ws);
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

void fill_meta(hq_qtensor* q, int64_t rows, int64_t cols, const hq_config* cfg, int32_t rot) {
  q->rows = rows;
  q->cols = cols;
  q->k = cfg->k;
  q->bits = cfg->bits;
  q->rot = rot;
  q->format = cfg->format;
}

hq_status check_saved(const hq_qtensor* q, int64_t rows, int64_t cols, const hq_config* cfg,
                      int32_t rot) {
  if (!q || !q->scale || (!q->codes_t && rows * cols > 0)) return HQ_ERR_NULL;
  if (q->rows != rows || q->cols != cols || q->k != cfg->k || q->bits != cfg->bits ||
      q->rot != rot || q->format != cfg->format)
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
    case HQ_ERR_BITS: return "bits must be 4 or 8 for integer codes, 8 for E4M3, 6 for E2M3 / E3M2";
    case HQ_ERR_DTYPE: return "unsupported dtype";
    case HQ_ERR_MODE: return "bad rotation, scale mode, variant or code format";
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
  HQ_CHECK(quantize_tensor(src, src_dtype, rows, cols, rot, cfg->k, cfg,
                           cfg->scale_mode == HQ_SCALE_STEP ? step : nullptr, out->codes,
                           out->ld, out->codes_t, out->ld_t, out->scale, w, 0, st));
  fill_meta(out, rows, cols, cfg, rot);
  return HQ_OK;
}

}  // extern "C"

namespace hq {

size_t fwd_workspace_bytes() { return ws_need(); }

// Argument checks of hq_linear_fwd (all but the workspace), before any HIP call. With
// batch > 1 (hq_bmm_fwd) X, W and Y are batch stacked N x C, D x C and N x D matrices: the
// codes describe the stacked (batch N) x C and (batch D) x C matrices, N and D must be
// multiples of 16 so that every batch's block of the transposed code layouts starts on a
// 16-byte boundary.
hq_status fwd_validate(const void* x, const void* w, int32_t in_dtype, int64_t batch, int64_t N,
                       int64_t C, int64_t D, const hq_config* cfg, const float* step_x,
                       const float* step_w, const float* step_xt, const void* y,
                       int32_t y_dtype, const hq_qtensor* save_x, const hq_qtensor* save_xt,
                       const hq_qtensor* save_w) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(in_dtype) || !valid_dt(y_dtype)) return HQ_ERR_DTYPE;
  if (N < 0 || C < 0 || D < 0 || batch < 1 || batch > 65535) return HQ_ERR_SHAPE;
  if (batch > 1 && (N % 16 || D % 16)) return HQ_ERR_SHAPE;
  const int64_t NB = batch * N, DB = batch * D;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HALO0 && C % k) return HQ_ERR_SHAPE;
  const bool want_xt = (v == HQ_VARIANT_HALO2) && save_xt != nullptr;
  if (want_xt && N % k) return HQ_ERR_SHAPE;
  const bool stepm = cfg->scale_mode == HQ_SCALE_STEP;
  if (stepm && (!step_x || !step_w || (want_xt && !step_xt))) return HQ_ERR_NULL;
  if ((NB * C > 0 && !x) || (DB * C > 0 && !w) || (NB * D > 0 && !y)) return HQ_ERR_NULL;
  HQ_CHECK(check_qt_out(save_x, true, true, NB * C));
  HQ_CHECK(check_qt_out(save_w, true, true, DB * C));
  HQ_CHECK(check_pitches(save_x, NB, C));
  HQ_CHECK(check_pitches(save_w, DB, C));
  if (want_xt) {
    if (!save_xt->scale || (!save_xt->codes_t && NB * C > 0)) return HQ_ERR_NULL;
    HQ_CHECK(check_pitches(save_xt, NB, C));
  }
  return HQ_OK;
}

// The launches of the forward on a validated call; ws holds at least fwd_workspace_bytes().
hq_status fwd_run(const void* x, const void* w, int32_t in_dtype, int64_t batch, int64_t Nb,
                  int64_t C, int64_t Db, const hq_config* cfg, const float* step_x,
                  const float* step_w, const float* step_xt, void* y, int32_t y_dtype,
                  hq_qtensor* save_x, hq_qtensor* save_xt, hq_qtensor* save_w, void* ws,
                  void* stream) {
  // the prologue quantizes the stacked matrices (one scale per batched tensor; right rotations
  // act within rows and token blocks of k rows never cross a batch); the product is batched
  const int64_t N = batch * Nb, D = batch * Db;
  const int32_t v = cfg->variant, k = cfg->k;
  const bool want_xt = (v == HQ_VARIANT_HALO2) && save_xt != nullptr;
  const bool stepm = cfg->scale_mode == HQ_SCALE_STEP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws wsp(ws);
  const int32_t rx = x_rot(v);
  const bool two_sided = want_xt && !save_x->codes_t && !save_xt->codes && k > 1;
  // X's two-sided pass runs in a single launch over a grid barrier when it is small enough;
  // W's quantize pass, launched just before, zeroes the barrier words
  hq::ProPass px;
  bool single = false;
  if (two_sided && !stepm && N * C > 0) {
    px = x_both_pass(x, in_dtype, N, C, k, cfg, nullptr, nullptr, save_x, save_xt, wsp);
    single = hq::pro_single_ok(px, device_info().cus) && D * C > 0;
  }
  HQ_CHECK(quantize_tensor(w, in_dtype, D, C, rx, k, cfg, stepm ? step_w : nullptr,
                           save_w->codes, save_w->ld, save_w->codes_t, save_w->ld_t,
                           save_w->scale, wsp, 2, st, single ? wsp.bar : nullptr,
                           single ? hq::kBarWordsInts : 0));
  fill_meta(save_w, D, C, cfg, rx);
  if (single) {
    px.nparts = hq::pro_grid(px);
    HQ_TRY(hq::pro_single_pass(px, wsp.bar, st));
    HQ_TRY(hq::pro_fixup_pass(px, wsp.bar, st));
  } else if (two_sided) {
    HQ_CHECK(quantize_x_both(x, in_dtype, N, C, k, cfg, stepm ? step_x : nullptr,
                             stepm ? step_xt : nullptr, save_x, save_xt, wsp, st));
  } else {
    HQ_CHECK(quantize_tensor(x, in_dtype, N, C, rx, k, cfg, stepm ? step_x : nullptr,
                             save_x->codes, save_x->ld, save_x->codes_t, save_x->ld_t,
                             save_x->scale, wsp, 0, st));
    if (want_xt)
      HQ_CHECK(quantize_tensor(x, in_dtype, N, C, HQ_ROT_BOTH, k, cfg,
                               stepm ? step_xt : nullptr, k > 1 ? nullptr : save_xt->codes,
                               save_xt->ld, save_xt->codes_t, save_xt->ld_t, save_xt->scale,
                               wsp, 1, st));
  }
  fill_meta(save_x, N, C, cfg, rx);
  if (want_xt) fill_meta(save_xt, N, C, cfg, HQ_ROT_BOTH);
  GemmPass g;
  g.cus = device_info().cus;
  g.f8 = is_f8(cfg);
  g.a = save_x->codes;
  g.lda = save_x->ld;
  g.b = save_w->codes;
  g.ldb = save_w->ld;
  g.M = Nb;
  g.N = Db;
  g.K = C;
  g.batch = static_cast<int>(batch);
  g.a_bstride = Nb * save_x->ld;
  g.b_bstride = Db * save_w->ld;
  g.c_bstride = Nb * Db;
  g.epi = hq::EPI_SCALE;
  g.c = y;
  g.ldc = Db;
  g.out_dt = y_dtype;
  g.sa = save_x->scale;
  g.sb = save_w->scale;
  g.kmul = (v == HQ_VARIANT_HALO0) ? 1.0f : 1.0f / static_cast<float>(k);
  HQ_TRY(hq::gemm_pass(g, st));
  return HQ_OK;
}

hq_status device_ready() { return device_ok(); }

}  // namespace hq

extern "C" {

hq_status hq_linear_fwd(const void* x, const void* w, int32_t in_dtype, int64_t N, int64_t C,
                        int64_t D, const hq_config* cfg, const float* step_x,
                        const float* step_w, const float* step_xt, void* y, int32_t y_dtype,
                        hq_qtensor* save_x, hq_qtensor* save_xt, hq_qtensor* save_w, void* ws,
                        size_t ws_bytes, void* stream) {
  HQ_CHECK(hq::fwd_validate(x, w, in_dtype, 1, N, C, D, cfg, step_x, step_w, step_xt, y,
                            y_dtype, save_x, save_xt, save_w));
  HQ_CHECK(check_ws(ws, ws_bytes, hq_workspace_bytes(cfg, N, C, D)));
  HQ_CHECK(device_ok());
  return hq::fwd_run(x, w, in_dtype, 1, N, C, D, cfg, step_x, step_w, step_xt, y, y_dtype,
                     save_x, save_xt, save_w, ws, stream);
}

}  // extern "C"

namespace {

// The input gradient of a layer (batch == 1) or of a batched product: dY is batch stacked
// N x D matrices, its codes describe the stacked (batch N) x D matrix, and the product runs per
// batch against the stacked transposed codes of W (batch D columns).
hq_status bwd_input_impl(const void* dy, int32_t dy_dtype, int64_t batch, int64_t N, int64_t C,
                         int64_t D, const hq_config* cfg, const float* step_g,
                         const hq_qtensor* saved_w, void* dx, int32_t dx_dtype,
                         hq_qtensor* save_g, void* ws, size_t ws_bytes, size_t ws_min,
                         void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(dy_dtype) || !valid_dt(dx_dtype)) return HQ_ERR_DTYPE;
  if (N < 0 || C < 0 || D < 0 || batch < 1 || batch > 65535) return HQ_ERR_SHAPE;
  if (batch > 1 && (N % 16 || D % 16)) return HQ_ERR_SHAPE;
  const int64_t NB = batch * N, DB = batch * D;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HALO0 && C % k) return HQ_ERR_SHAPE;
  if (v == HQ_VARIANT_HALO2 && N % k) return HQ_ERR_SHAPE;
  const bool stepm = cfg->scale_mode == HQ_SCALE_STEP;
  if (stepm && !step_g) return HQ_ERR_NULL;
  if ((NB * D > 0 && !dy) || (NB * C > 0 && !dx)) return HQ_ERR_NULL;
  HQ_CHECK(check_saved(saved_w, DB, C, cfg, x_rot(v)));
  HQ_CHECK(check_qt_out(save_g, true, true, NB * D));
  HQ_CHECK(check_pitches(save_g, NB, D));
  HQ_CHECK(check_ws(ws, ws_bytes, ws_min));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws wsp(ws);
  const int32_t rg = g_rot(v);
  // paired dX tiles need their arrival flags at zero: the quantize pass clears them
  const int64_t split = batch == 1 ? dx_split_tiles(cfg, N, C, D) : 0;
  HQ_CHECK(quantize_tensor(dy, dy_dtype, NB, D, rg, k, cfg, stepm ? step_g : nullptr,
                           save_g->codes, save_g->ld, save_g->codes_t, save_g->ld_t,
                           save_g->scale, wsp, 0, st,
                           split > 0 ? static_cast<int32_t*>(wsp.split) : nullptr, split));
  fill_meta(save_g, NB, D, cfg, rg);
  // dX = [B_N] (qG qW) [B_C] sG sW / k^e, dequantized and inverse-rotated in the GEMM epilogue.
  GemmPass g;
  g.cus = device_info().cus;
  g.f8 = is_f8(cfg);
  g.epi = hq::EPI_SCALE;
  g.sa = save_g->scale;
  g.sb = saved_w->scale;
  g.c = dx;
  g.out_dt = dx_dtype;
  g.ldc = C;
  g.K = D;
  g.batch = static_cast<int>(batch);
  g.c_bstride = N * C;
  if (v == HQ_VARIANT_HQ) {
    // only the columns (C) rotate: compute dX^T = qW^T qG^T so C is the tile's row axis,
    // where the epilogue rotates in registers, and store it transposed
    g.a = saved_w->codes_t;
    g.lda = saved_w->ld_t;
    g.a_bstride = D;                     // batch b: columns b D + [0, D) of the stacked qW^T
    g.b = save_g->codes;
    g.ldb = save_g->ld;
    g.b_bstride = N * save_g->ld;
    g.M = C;
    g.N = N;
    g.km = k;
    g.trans_out = true;
    g.kmul = 1.0f / static_cast<float>(k);
  } else {
    g.a = save_g->codes;
    g.lda = save_g->ld;
    g.a_bstride = N * save_g->ld;
    g.b = saved_w->codes_t;
    g.ldb = saved_w->ld_t;
    g.b_bstride = D;
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

// The weight gradient from saved codes only, of a layer or a batched product (the codes of
// dY and X describe stacked matrices; batch b contracts over its own N tokens).
hq_status bwd_weight_impl(const hq_qtensor* saved_g, const hq_qtensor* saved_x, int64_t batch,
                          int64_t N, int64_t C, int64_t D, const hq_config* cfg, void* dw,
                          int32_t dw_dtype, void* ws, size_t ws_bytes, size_t ws_min,
                          void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(dw_dtype)) return HQ_ERR_DTYPE;
  if (N < 0 || C < 0 || D < 0 || batch < 1 || batch > 65535) return HQ_ERR_SHAPE;
  if (batch > 1 && (N % 16 || D % 16)) return HQ_ERR_SHAPE;
  const int64_t NB = batch * N;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HALO0 && C % k) return HQ_ERR_SHAPE;
  if (v == HQ_VARIANT_HALO2 && N % k) return HQ_ERR_SHAPE;
  if (batch * D * C > 0 && !dw) return HQ_ERR_NULL;
  HQ_CHECK(check_saved(saved_g, NB, D, cfg, g_rot(v)));
  HQ_CHECK(check_saved(saved_x, NB, C, cfg, xt_rot(v)));
  HQ_CHECK(check_ws(ws, ws_bytes, ws_min));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  // dW = (qG^T qX') [B_C] sG sX' / k^e. When C rotates, compute dW^T = qX'^T qG so C is the
  // tile's row axis (rotated in registers) and store it transposed.
  GemmPass g;
  g.cus = device_info().cus;
  g.f8 = is_f8(cfg);
  g.epi = hq::EPI_SCALE;
  g.sa = saved_g->scale;
  g.sb = saved_x->scale;
  g.c = dw;
  g.out_dt = dw_dtype;
  g.ldc = C;
  g.K = N;
  g.batch = static_cast<int>(batch);
  g.a_bstride = N;                       // batch b: columns b N + [0, N) of both operands
  g.b_bstride = N;
  g.c_bstride = D * C;
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

}  // namespace

extern "C" {

hq_status hq_linear_bwd_input(const void* dy, int32_t dy_dtype, int64_t N, int64_t C, int64_t D,
                              const hq_config* cfg, const float* step_g,
                              const hq_qtensor* saved_w, void* dx, int32_t dx_dtype,
                              hq_qtensor* save_g, void* ws, size_t ws_bytes, void* stream) {
  const size_t need = cfg ? hq_workspace_bytes(cfg, N, C, D) : 0;
  return bwd_input_impl(dy, dy_dtype, 1, N, C, D, cfg, step_g, saved_w, dx, dx_dtype, save_g, ws,
                        ws_bytes, need, stream);
}

hq_status hq_linear_bwd_weight(const hq_qtensor* saved_g, const hq_qtensor* saved_x, int64_t N,
                               int64_t C, int64_t D, const hq_config* cfg, void* dw,
                               int32_t dw_dtype, void* ws, size_t ws_bytes, void* stream) {
  const size_t need = cfg ? hq_workspace_bytes(cfg, N, C, D) : 0;
  return bwd_weight_impl(saved_g, saved_x, 1, N, C, D, cfg, dw, dw_dtype, ws, ws_bytes, need,
                         stream);
}

size_t hq_bmm_workspace_bytes(const hq_config* cfg) {
  if (check_cfg(cfg) != HQ_OK) return 0;
  return ws_need();
}

hq_status hq_bmm_fwd(const void* x, const void* w, int32_t in_dtype, int64_t batch, int64_t N,
                     int64_t C, int64_t D, const hq_config* cfg, const float* step_x,
                     const float* step_w, const float* step_xt, void* y, int32_t y_dtype,
                     hq_qtensor* save_x, hq_qtensor* save_xt, hq_qtensor* save_w, void* ws,
                     size_t ws_bytes, void* stream) {
  HQ_CHECK(hq::fwd_validate(x, w, in_dtype, batch, N, C, D, cfg, step_x, step_w, step_xt, y,
                            y_dtype, save_x, save_xt, save_w));
  HQ_CHECK(check_ws(ws, ws_bytes, ws_need()));
  HQ_CHECK(device_ok());
  return hq::fwd_run(x, w, in_dtype, batch, N, C, D, cfg, step_x, step_w, step_xt, y, y_dtype,
                     save_x, save_xt, save_w, ws, stream);
}

hq_status hq_bmm_bwd_input(const void* dy, int32_t dy_dtype, int64_t batch, int64_t N, int64_t C,
                           int64_t D, const hq_config* cfg, const float* step_g,
                           const hq_qtensor* saved_w, void* dx, int32_t dx_dtype,
                           hq_qtensor* save_g, void* ws, size_t ws_bytes, void* stream) {
  return bwd_input_impl(dy, dy_dtype, batch, N, C, D, cfg, step_g, saved_w, dx, dx_dtype, save_g,
                        ws, ws_bytes, ws_need(), stream);
}

hq_status hq_bmm_bwd_weight(const hq_qtensor* saved_g, const hq_qtensor* saved_x, int64_t batch,
                            int64_t N, int64_t C, int64_t D, const hq_config* cfg, void* dw,
                            int32_t dw_dtype, void* ws, size_t ws_bytes, void* stream) {
  return bwd_weight_impl(saved_g, saved_x, batch, N, C, D, cfg, dw, dw_dtype, ws, ws_bytes,
                         ws_need(), stream);
}

}  // extern "C"

namespace {
hq_status check_stat_args(const void* src, const void* grad, int32_t dtype, int64_t rows,
                          int64_t cols, int32_t rot, const hq_config* cfg) {
  HQ_CHECK(check_cfg(cfg));
  if (!valid_dt(dtype)) return HQ_ERR_DTYPE;
  if (rot != HQ_ROT_NONE && rot != HQ_ROT_RIGHT) return HQ_ERR_MODE;
  if (rows < 0 || cols < 0) return HQ_ERR_SHAPE;
  if (rot == HQ_ROT_RIGHT && cols % cfg->k) return HQ_ERR_SHAPE;
  if (rows * cols > 0 && !src) return HQ_ERR_NULL;
  (void)grad;
  return HQ_OK;
}

hq::StatPass stat_pass_for(const void* src, const void* grad, int32_t dtype, int64_t rows,
                           int64_t cols, int32_t rot, const hq_config* cfg, int mode,
                           const Ws& w) {
  hq::StatPass p;
  p.src = src;
  p.grad = grad;
  p.dt = dtype;
  p.rows = rows;
  p.cols = cols;
  p.k = rot == HQ_ROT_RIGHT ? cfg->k : 1;
  p.mode = mode;
  p.f8 = is_f8(cfg);
  p.qp = qmax(cfg);
  p.partials = reinterpret_cast<double*>(w.part[0]);   // part[0..3]: kStatMaxParts doubles
  return p;
}
}  // namespace

extern "C" {

hq_status hq_rotated_stat(const void* src, const void* grad, int32_t dtype, int64_t rows,
                          int64_t cols, int32_t rot, const hq_config* cfg, int32_t stat,
                          const float* scale, double* out, void* ws, size_t ws_bytes,
                          void* stream) {
  HQ_CHECK(check_stat_args(src, grad, dtype, rows, cols, rot, cfg));
  if (stat != HQ_STAT_ABS_SUM && stat != HQ_STAT_QERR && stat != HQ_STAT_LSQ_GRAD)
    return HQ_ERR_MODE;
  if (stat == HQ_STAT_LSQ_GRAD && is_f8(cfg)) return HQ_ERR_MODE;
  if (stat == HQ_STAT_QERR && is_fp6(cfg)) return HQ_ERR_MODE;   // E4M3 and integer grids only
  if (stat == HQ_STAT_LSQ_GRAD && rows * cols > 0 && !grad) return HQ_ERR_NULL;
  if (stat != HQ_STAT_ABS_SUM && !scale) return HQ_ERR_NULL;
  if (!out) return HQ_ERR_NULL;
  HQ_CHECK(check_ws(ws, ws_bytes, ws_need()));
  HQ_CHECK(device_ok());
  Ws w(ws);
  hq::StatPass p = stat_pass_for(src, grad, dtype, rows, cols, rot, cfg, stat, w);
  p.scale = scale;
  p.out = out;
  HQ_TRY(hq::stat_pass(p, static_cast<hipStream_t>(stream)));
  return HQ_OK;
}

hq_status hq_cold_start_step(const void* src, int32_t dtype, int64_t rows, int64_t cols,
                             int32_t rot, const hq_config* cfg, float* step, void* ws,
                             size_t ws_bytes, void* stream) {
  HQ_CHECK(check_stat_args(src, nullptr, dtype, rows, cols, rot, cfg));
  if (is_f8(cfg)) return HQ_ERR_MODE;
  if (!step) return HQ_ERR_NULL;
  if (rows * cols == 0) return HQ_ERR_SHAPE;   // no entries: no mean to set a step from
  HQ_CHECK(check_ws(ws, ws_bytes, ws_need()));
  HQ_CHECK(device_ok());
  Ws w(ws);
  hq::StatPass p = stat_pass_for(src, nullptr, dtype, rows, cols, rot, cfg, HQ_STAT_ABS_SUM, w);
  p.finish = 2;
  p.fout = step;
  HQ_TRY(hq::stat_pass(p, static_cast<hipStream_t>(stream)));
  return HQ_OK;
}

hq_status hq_select_hadamard_k(const void* x, const void* w, int32_t dtype, int64_t N, int64_t C,
                               int64_t D, const hq_config* cfg, const int32_t* candidates,
                               int32_t n_candidates, int32_t* k_best, double* errors, void* ws,
                               size_t ws_bytes, void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (is_fp6(cfg)) return HQ_ERR_MODE;   // error passes on the E4M3 and integer grids only
  if (!valid_dt(dtype)) return HQ_ERR_DTYPE;
  if (N <= 0 || C <= 0 || D <= 0) return HQ_ERR_SHAPE;
  if (!x || !w || !candidates || !k_best) return HQ_ERR_NULL;
  if (n_candidates < 1 || n_candidates > HQ_MAX_K_CANDIDATES) return HQ_ERR_SHAPE;
  for (int32_t i = 0; i < n_candidates; ++i) {
    if (!is_pow2_k(candidates[i])) return HQ_ERR_K;
    if (C % candidates[i]) return HQ_ERR_SHAPE;
  }
  HQ_CHECK(check_ws(ws, ws_bytes, ws_need()));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws wsp(ws);
  // results in the grid-barrier words (unused by these passes; the partials take part[0..3])
  static_assert(2 * HQ_MAX_K_CANDIDATES * sizeof(double) + 2 * sizeof(float) + kAlign <= kBarBytes,
                "selection results fit the barrier words");
  double* res = reinterpret_cast<double*>(wsp.bar);                              // 2 per candidate
  float* sc = reinterpret_cast<float*>(reinterpret_cast<char*>(wsp.bar) + kAlign);   // 2 scales
  hq_config c = *cfg;
  for (int32_t i = 0; i < n_candidates; ++i) {
    c.k = candidates[i];
    for (int t = 0; t < 2; ++t) {
      const void* src = t == 0 ? x : w;
      const int64_t rows = t == 0 ? N : D;
      hq::StatPass p = stat_pass_for(src, nullptr, dtype, rows, C, HQ_ROT_RIGHT, &c,
                                     hq::STAT_MODE_ABS_MAX, wsp);
      p.finish = 1;
      p.fout = sc + t;
      HQ_TRY(hq::stat_pass(p, st));
      p = stat_pass_for(src, nullptr, dtype, rows, C, HQ_ROT_RIGHT, &c, HQ_STAT_QERR, wsp);
      p.scale = sc + t;
      p.out = res + 2 * i + t;
      HQ_TRY(hq::stat_pass(p, st));
    }
  }
  double host[2 * HQ_MAX_K_CANDIDATES];
  HQ_TRY(hipMemcpyAsync(host, res, sizeof(double) * 2 * n_candidates, hipMemcpyDeviceToHost, st));
  HQ_TRY(hipStreamSynchronize(st));
  int32_t best = -1;
  double best_prod = 0.0;
  for (int32_t i = 0; i < n_candidates; ++i) {
    // errors in the space of X and W: ||V - s Q(V B) B / k||^2 = sum (v - s q)^2 / k
    const double ex = host[2 * i] / candidates[i], ew = host[2 * i + 1] / candidates[i];
    if (errors) {
      errors[2 * i] = ex;
      errors[2 * i + 1] = ew;
    }
    if (best < 0 || ex * ew < best_prod) {
      best = i;
      best_prod = ex * ew;
    }
  }
  *k_best = candidates[best];
  return HQ_OK;
}

hq_status hq_fwht_path(const void* src, int32_t src_dtype, void* dst, int32_t dst_dtype,
                       int64_t rows, int64_t cols, int32_t rot, int32_t k, int32_t path,
                       void* stream) {
  if (!valid_dt(src_dtype) || !valid_dt(dst_dtype)) return HQ_ERR_DTYPE;
  if (!is_pow2_k(k)) return HQ_ERR_K;
  if (rot != HQ_ROT_NONE && rot != HQ_ROT_RIGHT && rot != HQ_ROT_LEFT) return HQ_ERR_MODE;
  if (path != HQ_FWHT_AUTO && path != HQ_FWHT_BUTTERFLY && path != HQ_FWHT_MATRIX)
    return HQ_ERR_MODE;
  if (rows < 0 || cols < 0) return HQ_ERR_SHAPE;
  if (rot == HQ_ROT_RIGHT && cols % k) return HQ_ERR_SHAPE;
  if (rot == HQ_ROT_LEFT && rows % k) return HQ_ERR_SHAPE;
  if (rows * cols > 0 && (!src || !dst)) return HQ_ERR_NULL;
  // the matrix-core store kernels cover whole tiles of 16-bit data only (see hq.h)
  const bool left_mma = rot == HQ_ROT_LEFT && k >= 16 &&
                        hq::fwht_left_mma_ok(src, src_dtype, dst, dst_dtype, rows, cols, k);
  const bool right_mma = rot == HQ_ROT_RIGHT && k >= 16 &&
                         hq::fwht_right_mma_ok(src, src_dtype, dst, dst_dtype, rows, cols, k);
  if (path == HQ_FWHT_MATRIX && !left_mma && !right_mma) return HQ_ERR_MODE;
  if (rows * cols == 0) return HQ_OK;
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  // AUTO follows the measured bf16 transforms (2048 x 4096 up to 8192 x 13824): the
  // butterflies wherever they are within 5 % of the matrix cores (RIGHT at every k; LEFT up
  // to k = 128, with non-temporal output stores 65-88 us against 97 us), the matrix cores
  // otherwise (LEFT at k = 256: 97 against 113 us)
  const bool auto_left_mma = k >= 256;
  const bool auto_right_mma = false;
  const bool use_left_mma =
      left_mma && (path == HQ_FWHT_MATRIX || (path == HQ_FWHT_AUTO && auto_left_mma));
  const bool use_right_mma =
      right_mma && (path == HQ_FWHT_MATRIX || (path == HQ_FWHT_AUTO && auto_right_mma));
  if (use_left_mma) {
    HQ_TRY(hq::fwht_left_mma(src, src_dtype, rows, cols, k, dst, st));
    return HQ_OK;
  }
  if (use_right_mma) {
    HQ_TRY(hq::fwht_right_mma(src, src_dtype, rows, cols, k, dst, st));
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

hq_status hq_fwht(const void* src, int32_t src_dtype, void* dst, int32_t dst_dtype, int64_t rows,
                  int64_t cols, int32_t rot, int32_t k, void* stream) {
  return hq_fwht_path(src, src_dtype, dst, dst_dtype, rows, cols, rot, k, HQ_FWHT_AUTO, stream);
}

}  // extern "C"

namespace {
hq_status gemm_plain(const void* a, int64_t lda, const void* b_t, int64_t ldb, void* c,
                     int64_t M, int64_t N, int64_t K, bool f8, void* stream) {
  if (M < 0 || N < 0 || K < 0) return HQ_ERR_SHAPE;
  if ((M * K > 0 && !a) || (N * K > 0 && !b_t) || (M * N > 0 && !c)) return HQ_ERR_NULL;
  if (lda < K || ldb < K) return HQ_ERR_SHAPE;
  if (lda % 16 || ldb % 16 || (a && !aligned16(a)) || (b_t && !aligned16(b_t))) return HQ_ERR_ALIGN;
  if (M * N == 0) return HQ_OK;
  HQ_CHECK(device_ok());
  GemmPass g;
  g.cus = device_info().cus;
  g.f8 = f8;
  g.a = static_cast<const int8_t*>(a);
  g.lda = lda;
  g.b = static_cast<const int8_t*>(b_t);
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
}  // namespace

extern "C" {

hq_status hq_gemm_f8_f32(const uint8_t* a, int64_t lda, const uint8_t* b_t, int64_t ldb, float* c,
                         int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_plain(a, lda, b_t, ldb, c, M, N, K, true, stream);
}

hq_status hq_gemm_i8_i32(const int8_t* a, int64_t lda, const int8_t* b_t, int64_t ldb,
                         int32_t* c, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_plain(a, lda, b_t, ldb, c, M, N, K, false, stream);
}

}  // extern "C"

namespace {
// LSS-MM workspace: absmax partials, the stats record, then per-token arrays (row maxima,
// scores, probabilities, clamp flags, kept list) and the two K-contiguous GEMM operands.
constexpr int64_t kLssMaxN = int64_t(1) << 21;   // int32 sums of the combined-code product
constexpr int64_t kLssMaxDim = int64_t(1) << 20;   // pack grid: (C + D) / 64 rows of tiles

struct LssWs {
  float* partials;
  hq_lss_stats* stats;
  float* rowmax;
  double* scores;
  double* probs;
  uint8_t* fixed;
  int32_t* kept_idx;
  double* kept_p;
  int8_t* ct;
  int8_t* xt;
  int64_t ldk;
  size_t bytes;
  LssWs(void* base, int64_t N, int64_t C, int64_t D) {
    char* b = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t n) {
      char* p = b ? b + off : nullptr;
      off = align_up(off + n, kAlign);
      return p;
    };
    ldk = pitch16(N);
    partials = reinterpret_cast<float*>(take(hq::kMaxPartials * sizeof(float)));
    stats = reinterpret_cast<hq_lss_stats*>(take(sizeof(hq_lss_stats)));
    rowmax = reinterpret_cast<float*>(take(N * sizeof(float)));
    scores = reinterpret_cast<double*>(take(N * sizeof(double)));
    probs = reinterpret_cast<double*>(take(N * sizeof(double)));
    fixed = reinterpret_cast<uint8_t*>(take(N));
    kept_idx = reinterpret_cast<int32_t*>(take(N * sizeof(int32_t)));
    kept_p = reinterpret_cast<double*>(take(N * sizeof(double)));
    ct = reinterpret_cast<int8_t*>(take(D * ldk));
    xt = reinterpret_cast<int8_t*>(take(C * ldk));
    bytes = off;
  }
};

bool lss_dims_ok(int64_t N, int64_t C, int64_t D) {
  return N >= 0 && C >= 0 && D >= 0 && N <= kLssMaxN && C <= kLssMaxDim && D <= kLssMaxDim;
}
}  // namespace

extern "C" {

size_t hq_lss_workspace_bytes(int64_t N, int64_t C, int64_t D) {
  if (!lss_dims_ok(N, C, D)) return 0;
  return LssWs(nullptr, N, C, D).bytes;
}

hq_status hq_lss_bwd_weight(const void* dy, int32_t dy_dtype, const hq_qtensor* saved_x,
                            int64_t N, int64_t C, int64_t D, const hq_config* cfg, double budget,
                            const float* uniforms, void* dw, int32_t dw_dtype, double* probs,
                            int32_t* kept_idx, hq_lss_stats* stats, void* ws, size_t ws_bytes,
                            void* stream) {
  HQ_CHECK(check_cfg(cfg));
  if (cfg->format != HQ_FMT_INT) return HQ_ERR_MODE;
  if (cfg->bits != 4) return HQ_ERR_BITS;
  const int32_t v = cfg->variant, k = cfg->k;
  if (v != HQ_VARIANT_HQ && v != HQ_VARIANT_HALO0) return HQ_ERR_MODE;
  if (!valid_dt(dy_dtype) || !valid_dt(dw_dtype)) return HQ_ERR_DTYPE;
  if (!lss_dims_ok(N, C, D)) return HQ_ERR_SHAPE;
  if (v == HQ_VARIANT_HQ && C % k) return HQ_ERR_SHAPE;
  if (!std::isfinite(budget)) return HQ_ERR_SHAPE;
  if (N * D > 0 && !dy) return HQ_ERR_NULL;
  if (N > 0 && !uniforms) return HQ_ERR_NULL;
  if (D * C > 0 && !dw) return HQ_ERR_NULL;
  if (!saved_x || !saved_x->scale || (N * C > 0 && !saved_x->codes)) return HQ_ERR_NULL;
  if (saved_x->rows != N || saved_x->cols != C || saved_x->k != k || saved_x->bits != cfg->bits ||
      saved_x->rot != x_rot(v) || saved_x->format != cfg->format)
    return HQ_ERR_MISMATCH;
  if (saved_x->codes && (!aligned16(saved_x->codes) || saved_x->ld % 16)) return HQ_ERR_ALIGN;
  if (saved_x->codes && saved_x->ld < C) return HQ_ERR_SHAPE;
  if ((probs && !aligned16(probs)) || (kept_idx && !aligned16(kept_idx)) ||
      (stats && !aligned16(stats)))
    return HQ_ERR_ALIGN;
  const LssWs need(nullptr, N, C, D);
  HQ_CHECK(check_ws(ws, ws_bytes, need.bytes));
  HQ_CHECK(device_ok());
  hipStream_t st = static_cast<hipStream_t>(stream);
  LssWs w(ws, N, C, D);
  hq::LssPass p;
  p.dy = dy;
  p.dt = dy_dtype;
  p.N = N;
  p.C = C;
  p.D = D;
  p.qx = saved_x->codes;
  p.ldx = saved_x->ld;
  p.budget = budget;
  p.uniforms = uniforms;
  p.partials = w.partials;
  p.rowmax = w.rowmax;
  p.scores = w.scores;
  p.probs = probs ? probs : w.probs;
  p.fixed = w.fixed;
  p.kept_idx = kept_idx ? kept_idx : w.kept_idx;
  p.kept_p = w.kept_p;
  p.stats = stats ? stats : w.stats;
  p.ct = w.ct;
  p.xt = w.xt;
  p.ldk = w.ldk;
  HQ_TRY(hq::lss_pass(p, st));
  // dW = (14 hi + lo)^T qX_kept [B_C] s_lo sX / k over the K' kept tokens; with B_C the
  // transpose dW^T = qX_kept^T (14 hi + lo) is formed so C is the tile's rotated row axis
  GemmPass g;
  g.cus = device_info().cus;
  g.epi = hq::EPI_SCALE;
  g.sa = &p.stats->s_lo;
  g.sb = saved_x->scale;
  g.c = dw;
  g.out_dt = dw_dtype;
  g.ldc = C;
  g.K = N;
  g.k_dev = &p.stats->kept;
  if (v == HQ_VARIANT_HALO0) {
    g.a = w.ct;
    g.lda = w.ldk;
    g.b = w.xt;
    g.ldb = w.ldk;
    g.M = D;
    g.N = C;
  } else {
    g.a = w.xt;
    g.lda = w.ldk;
    g.b = w.ct;
    g.ldb = w.ldk;
    g.M = C;
    g.N = D;
    g.km = k;
    g.trans_out = true;
    g.kmul = 1.0f / static_cast<float>(k);
  }
  HQ_TRY(hq::gemm_pass(g, st));
  return HQ_OK;
}

}  // extern "C"
