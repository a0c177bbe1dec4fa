// Stand-ins for the kernel launchers of libhq (defined in the .hip files), for the host-only
// AddressSanitizer / UndefinedBehaviorSanitizer build of the C-ABI layer (hq_api.cpp,
// hq_profile.cpp). That build runs the argument checks only: every call it is given fails
// validation, or reaches the device check and fails there on a machine without a GPU, so no
// launcher below is ever reached. Each reports a launch failure if one were.
#include "../../hadamard_rotated_precision_amd/csrc/hq_internal.hpp"

namespace hq {

int pro_grid(const ProPass&) { return 1; }
hipError_t pro_pass(const ProPass&, int, hipStream_t) { return hipErrorInvalidValue; }
bool pro_single_ok(const ProPass&, int) { return false; }
hipError_t pro_single_pass(const ProPass&, int32_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t pro_fixup_pass(const ProPass&, int32_t*, hipStream_t) { return hipErrorInvalidValue; }
bool fwht_right_mma_ok(const void*, int, const void*, int, int64_t, int64_t, int) { return false; }
hipError_t fwht_right_mma(const void*, int, int64_t, int64_t, int, void*, hipStream_t) {
  return hipErrorInvalidValue;
}
bool fwht_left_mma_ok(const void*, int, const void*, int, int64_t, int64_t, int) { return false; }
hipError_t fwht_left_mma(const void*, int, int64_t, int64_t, int, void*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t rows_pass(const RowPass&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t stat_pass(const StatPass&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t cols_pass(const ColPass&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t write_scale(float*, const float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t gemm_pass(const GemmPass&, hipStream_t) { return hipErrorInvalidValue; }
int64_t gemm_split_tiles(int64_t, int64_t, int64_t, int, int, int, bool) { return 0; }
size_t gemm_split_bytes(int64_t) { return 0; }
hipError_t zero_i32(int32_t*, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t lss_pass(const LssPass&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace hq

// The no-allocation forward (hq_static.hip) up to its device check: the same argument checks.
extern "C" hq_status hq_linear_fwd_noalloc(const void* x, const void* w, int32_t in_dtype,
                                           int64_t N, int64_t C, int64_t D,
                                           const hq_config* cfg, const float* step_x,
                                           const float* step_w, const float* step_xt, void* y,
                                           int32_t y_dtype, hq_qtensor* save_x,
                                           hq_qtensor* save_xt, hq_qtensor* save_w, void*) {
  hq_status s = hq::fwd_validate(x, w, in_dtype, 1, N, C, D, cfg, step_x, step_w, step_xt, y,
                                 y_dtype, save_x, save_xt, save_w);
  if (s != HQ_OK) return s;
  if (hq::fwd_workspace_bytes() > 20 * 1024) return HQ_ERR_WORKSPACE;
  return hq::device_ready();
}
