// hq_internal.hpp — launchers shared between the kernel files and the C-ABI layer of libhq
// (plain host C++: the kernel files add hq_launch.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hq.h"

namespace hq {

// The forward of hq_linear_fwd in two halves (hq_api.cpp), shared with the entry point that
// brings its own scratch: fwd_validate runs every argument check except the workspace's;
// fwd_run launches the passes on a validated call with a workspace of at least
// fwd_workspace_bytes() bytes. device_ready: HQ_OK when the current device is usable.
// batch > 1: the batched product of hq_bmm_fwd (N and D per batch).
size_t fwd_workspace_bytes();
hq_status fwd_validate(const void* x, const void* w, int32_t in_dtype, int64_t batch, int64_t N,
                       int64_t C, int64_t D, const hq_config* cfg, const float* step_x,
                       const float* step_w, const float* step_xt, const void* y,
                       int32_t y_dtype, const hq_qtensor* save_x, const hq_qtensor* save_xt,
                       const hq_qtensor* save_w);
hq_status fwd_run(const void* x, const void* w, int32_t in_dtype, int64_t batch, int64_t N,
                  int64_t C, int64_t D, const hq_config* cfg, const float* step_x,
                  const float* step_w, const float* step_xt, void* y, int32_t y_dtype,
                  hq_qtensor* save_x, hq_qtensor* save_xt, hq_qtensor* save_w, void* ws,
                  void* stream);
hq_status device_ready();

// OP_STORE: the transform alone, rotated values written in the input dtype (hq_fwht).
// OP_QUANT_F8: the quantize pass writing FP8 E4M3 codes (pro_pass picks it from ProPass::f8);
// the format is a compile-time choice so each kernel carries one quantizer.
enum Op : int { OP_ABSMAX = 0, OP_QUANT = 1, OP_STORE = 2, OP_QUANT_F8 = 3 };

// Most partial maxima one absmax pass writes (its grid is capped to this).
constexpr int kMaxPartials = 1024;

// The standalone transform (hq_rotate.hip): rotate a rows x cols matrix along the contiguous
// axis (rows_pass; k = 1 copies with a dtype conversion) or along the row axis in k-row blocks
// (cols_pass), writing the rotated values in out_dt.
struct RowPass {
  const void* src = nullptr;
  int in_dt = 0;
  int64_t rows = 0, cols = 0;
  int k = 1;            // 1 = no rotation
  void* dst = nullptr;
  int out_dt = 0;
};

struct ColPass {
  const void* src = nullptr;
  int in_dt = 0;
  int64_t rows = 0, cols = 0;   // rows % k == 0
  int k = 2;
  void* dst = nullptr;
  int out_dt = 0;
};

// Rotate -> scale -> quantize prologue (hq_prologue.hip).
enum ProKind : int { PRO_RIGHT = 0, PRO_LEFT = 1, PRO_BOTH = 2 };
struct ProPass {
  int kind = PRO_RIGHT;
  const void* src = nullptr;
  int in_dt = 0;
  int64_t rows = 0, cols = 0;
  int k = 1;                         // 1 with PRO_RIGHT = no rotation
  int qp = 127;                      // integer codes: the grid bound
  bool f8 = false;                   // float-format codes (E4M3 bytes) instead of integer codes
  float qmaxf = 127.0f;              // the scale's divisor: Qp, or the format's largest value
  int fgrid = 0;                     // f8: 0 E4M3, 1 E2M3, 2 E3M2 (FP6 values as E4M3 bytes)
  float* partials = nullptr;         // kMaxPartials floats
  int nparts = 0;                    // QUANT: grid of the ABSMAX pass (pro_grid)
  const float* step = nullptr;       // STEP mode (PRO_BOTH: step of X B)
  const float* step2 = nullptr;      // PRO_BOTH, STEP mode: step of B X B
  float* scale_out = nullptr;        // PRO_BOTH: scale of X B
  float* scale_out2 = nullptr;       // PRO_BOTH: scale of B X B
  int8_t* codes = nullptr;           // row-major codes (PRO_BOTH: of X B)
  int64_t ld = 0;
  int8_t* codes_t = nullptr;         // transposed codes (PRO_BOTH: of B X B; required)
  int64_t ld_t = 0;
  int32_t* zero_ptr = nullptr;       // QUANT pass also zeroes these ints (for a later launch)
  int64_t zero_n = 0;
};
int pro_grid(const ProPass& p);
hipError_t pro_pass(const ProPass& p, int op, hipStream_t st);
// Single-pass two-sided quantization (PRO_BOTH, ABSMAX mode, at most 256 half-tile items and
// no more than the device's `cus` compute units, since each item's workgroup takes a whole
// CU and all of them must be resident at once): pro_single_pass does both passes in one launch over a grid barrier in `bar` (kBarWordsInts
// ints, zeroed by an earlier launch on the stream); pro_fixup_pass, launched right after,
// recomputes the codes only if the single pass gave up waiting, and otherwise returns at once.
// The partials go to p.partials (2 x items floats); p.nparts must be pro_grid(p) (= items).
constexpr int kBarWordsInts = 512;
bool pro_single_ok(const ProPass& p, int cus);
hipError_t pro_single_pass(const ProPass& p, int32_t* bar, hipStream_t st);
hipError_t pro_fixup_pass(const ProPass& p, int32_t* bar, hipStream_t st);

// hq_fwht on the matrix cores, 16-bit in = out dtype: when fwht_right_mma_ok /
// fwht_left_mma_ok, one launch of the right / left prologue kernel in OP_STORE mode.
bool fwht_right_mma_ok(const void* src, int dt, const void* dst, int out_dt, int64_t rows,
                       int64_t cols, int k);
hipError_t fwht_right_mma(const void* src, int dt, int64_t rows, int64_t cols, int k, void* dst,
                          hipStream_t st);
bool fwht_left_mma_ok(const void* src, int dt, const void* dst, int out_dt, int64_t rows,
                      int64_t cols, int k);
hipError_t fwht_left_mma(const void* src, int dt, int64_t rows, int64_t cols, int k, void* dst,
                         hipStream_t st);
hipError_t rows_pass(const RowPass& p, hipStream_t st);

// Statistics of a right-rotated tensor (hq_rotate.hip, stat_kernel): mode is a StatMode
// (0 sum |v|, 1 sum (v - s q)^2, 2 LSQ step gradient, 3 max |v|); the reduced value goes to
// out (device double, or nullptr), and finish 1 / 2 also writes the absmax scale / cold-start
// step to fout. partials: kStatMaxParts doubles of workspace (the 16 KiB of absmax partials).
constexpr int kStatMaxParts = 2048;
constexpr int STAT_MODE_ABS_MAX = 3;
struct StatPass {
  const void* src = nullptr;
  const void* grad = nullptr;
  int dt = 0;
  int64_t rows = 0, cols = 0;
  int k = 1;
  int mode = 0;
  bool f8 = false;
  int qp = 127;
  const float* scale = nullptr;
  double* partials = nullptr;
  double* out = nullptr;
  int finish = 0;
  float* fout = nullptr;
};
hipError_t stat_pass(const StatPass& p, hipStream_t st);
hipError_t cols_pass(const ColPass& p, hipStream_t st);
hipError_t write_scale(float* scale, const float* step, hipStream_t st);

// LSS-MM sampling and bit split (hq_lss.hip): rowmax, score, probability and pack passes, up
// to the K-contiguous operands of the sampled weight-gradient GEMM (ct: D x ldk split codes,
// xt: C x ldk gathered X codes, K' = stats->kept columns valid, zeros up to the next multiple
// of 16). Buffers of N entries each; partials: kMaxPartials floats.
struct LssPass {
  const void* dy = nullptr;
  int dt = 0;
  int64_t N = 0, C = 0, D = 0;
  const int8_t* qx = nullptr;   // row-major X codes, pitch ldx
  int64_t ldx = 0;
  double budget = 0.0;
  const float* uniforms = nullptr;
  float* partials = nullptr;
  float* rowmax = nullptr;
  double* scores = nullptr;
  double* probs = nullptr;
  uint8_t* fixed = nullptr;
  int32_t* kept_idx = nullptr;
  double* kept_p = nullptr;     // probability of each kept token, in kept order
  hq_lss_stats* stats = nullptr;
  int8_t* ct = nullptr;
  int8_t* xt = nullptr;
  int64_t ldk = 0;
};
hipError_t lss_pass(const LssPass& p, hipStream_t st);

// Integer GEMM c = a * b^T (a: M x K, b: N x K, int8, K-contiguous) with int32 accumulation,
// or (f8) the product of FP8 E4M3 code matrices with fp32 accumulation.
enum Epi : int { EPI_I32 = 0, EPI_SCALE = 1 };
struct GemmPass {
  const int8_t* a = nullptr;
  int64_t lda = 0;
  const int8_t* b = nullptr;
  int64_t ldb = 0;
  int64_t M = 0, N = 0, K = 0;
  int epi = EPI_I32;
  void* c = nullptr;       // M x N, pitch ldc elements
  int64_t ldc = 0;
  int out_dt = 0;          // EPI_SCALE: output dtype
  const float* sa = nullptr;   // EPI_SCALE: alpha = (*sa * *sb) * kmul
  const float* sb = nullptr;
  float kmul = 1.0f;
  int km = 1;              // EPI_SCALE: inverse rotation block along M (rows), 1 = none
  int kn = 1;              // EPI_SCALE: along N (columns); km == kn when both are set
  bool trans_out = false;  // EPI_SCALE: store c^T (N x M, pitch ldc); requires kn == 1
  void* split_ws = nullptr;       // tile-pair workspace (gemm_split_bytes) when pairing applies
  bool split_cnt_zeroed = false;  // its arrival flags were zeroed by an earlier launch on the stream
  int cus = 0;             // compute units of the device (0: assume 256), for the tile rounds
  bool f8 = false;         // operands are FP8 E4M3 codes (fp32 accumulation; EPI_I32 stores fp32)
  int batch = 1;           // batched product: batch b reads a + b a_bstride, b + b b_bstride
  int64_t a_bstride = 0, b_bstride = 0;   // (bytes) and writes c + b c_bstride (elements)
  int64_t c_bstride = 0;
  const int32_t* k_dev = nullptr;   // contraction length written on the device (<= K), or none
};
hipError_t gemm_pass(const GemmPass& p, hipStream_t st);
// Number of tile pairs of a GEMM whose 256-wide column rotation spans two 256 x 128 tiles
// (0: none). Pairing is taken when 256-wide tiles would leave most CUs idle; the two tiles of a
// pair exchange their rotated values through the workspace and one of them finishes both.
int64_t gemm_split_tiles(int64_t M, int64_t N, int64_t K, int epi, int km, int kn, bool trans_out);
size_t gemm_split_bytes(int64_t pairs);
hipError_t zero_i32(int32_t* p, int64_t n, hipStream_t st);

// Launch instrumentation (hq_profile.cpp): returns a token, or -1 when not recording.
// prof_begin / prof_end bracket a launch with two event records on the stream; prof_open
// only takes the two events, which launch_k passes to hipExtLaunchKernel.
int prof_begin(int kind, double units, hipStream_t st);
void prof_end(int token, hipStream_t st);
int prof_open(int kind, double units);
void prof_events(int token, hipEvent_t* start, hipEvent_t* stop);

enum Kind : int { K_GEMM = 0, K_ROT_ABSMAX = 1, K_ROT_QUANT = 2, K_ROT_STORE = 3,
                  K_TRANSPOSE = 4, K_MISC = 5 };

}  // namespace hq
