// hq_static.hip — hq_linear_fwd_noalloc: the forward of hq_linear_fwd with its workspace taken
// from a fixed device array of this library instead of the caller's buffer, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). The kernels and the order of passes are those of hq_linear_fwd.
//
// The forward's workspace holds the per-workgroup absmax partials of the quantize passes and
// the grid-barrier words of the single-pass two-sided kernel (hq_api.cpp), about 18.7 KiB for
// any shape. Every piece of it is written before it is read within one call (the partials by
// the absmax pass, the barrier words by W's quantize pass), so nothing needs clearing between
// calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hq_internal.hpp"

namespace {

constexpr size_t kScratchBytes = 20 * 1024;

// One copy per device, held until the process ends. In host code this name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each device

// The device address of the current device's scratch array, looked up once per device with
// that device current.
hq_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HQ_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HQ_OK;
}

}  // namespace

extern "C" hq_status hq_linear_fwd_noalloc(const void* x, const void* w, int32_t in_dtype,
                                           int64_t N, int64_t C, int64_t D,
                                           const hq_config* cfg, const float* step_x,
                                           const float* step_w, const float* step_xt, void* y,
                                           int32_t y_dtype, hq_qtensor* save_x,
                                           hq_qtensor* save_xt, hq_qtensor* save_w,
                                           void* stream) {
  hq_status s = hq::fwd_validate(x, w, in_dtype, 1, N, C, D, cfg, step_x, step_w, step_xt, y,
                                 y_dtype, save_x, save_xt, save_w);
  if (s != HQ_OK) return s;
  if (hq::fwd_workspace_bytes() > kScratchBytes) return HQ_ERR_WORKSPACE;
  s = hq::device_ready();
  if (s != HQ_OK) return s;
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != HQ_OK) return s;
  return hq::fwd_run(x, w, in_dtype, 1, N, C, D, cfg, step_x, step_w, step_xt, y, y_dtype,
                     save_x, save_xt, save_w, ws, stream);
}
