/*
 * hq.h — C ABI of the MI355X (gfx950) Hadamard-quantized linear-layer library (libhq.so).
 *
 * What the library computes (cited by page title and section):
 *   "Training Transformers with 4-bit Integers" (paperlayer summary page):
 *     §3.1  learned-step quantizer mapping floating-point matrices to integers, INT4 range with
 *           Q_N = Q_P = 7, INT32 product dequantized back to floating point;
 *     §3.3  Hadamard quantization: block-diagonal transform with H_k blocks spreads outliers;
 *           the product is preserved because the transforms cancel (H H^T = k I);
 *     §4    backward reuses the forward-quantized activations and weights and quantizes the
 *           output gradient;
 *     §A.6  HQ-MM = Hadamard multiplication, quantization, packing, integer GEMM,
 *           dequantization; the integer GEMM wants both operands contiguous along K.
 *   "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs" (scime summary page):
 *     Problem   all three matmuls of a linear layer run in low precision;
 *     Approach  right-hand rotations of weights and activations in the forward pass, a
 *               left-hand (token-axis) rotation of output gradients in the backward pass
 *               (HALO-2), tensor-wise quantization, quantized rotated tensors reused;
 *     Limitations  tensor-wise round-to-nearest quantization.
 *
 * Shapes: X is N x C (N tokens, C in-features), W is D x C, dY is N x D, all row-major and
 * contiguous. Y = X W^T (N x D), dX = dY W (N x C), dW = dY^T X (D x C).
 *
 * Conventions that hold for every entry point:
 *   - Pointers are DEVICE pointers unless a comment says otherwise; device pointers must be
 *     16-byte aligned (HQ_ERR_ALIGN otherwise), except hq_fwht's src and dst, which need only
 *     the alignment of their element type.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream). Scales stay on the device; no call synchronizes with the host, except
 *     hq_select_hadamard_k, whose choice is made on the host.
 *   - Ownership: the caller allocates every buffer (codes, scales, outputs, workspace).
 *     The library allocates and frees nothing and keeps no pointer after it returns. Buffers
 *     must stay alive until the stream has reached the work.
 *   - Errors: all argument checks run before any launch; on error nothing is launched or
 *     written. A failed launch returns HQ_ERR_LAUNCH. Device faults surface at the caller's
 *     next synchronization.
 *   - Concurrency: stateless and reentrant; calls on different streams must use different
 *     workspaces and outputs.
 *   - Numerics: inputs must be finite. H is the unnormalized Sylvester matrix in natural
 *     order, h(i,j) = (-1)^popcount(i&j); its 1/k factors go into the dequantization scalar.
 *   - Environment switches, read on every call, for measuring one implementation against
 *     another (the results agree bit for bit unless noted): HQ_PROLOGUE_VALU=1 runs the
 *     rotate-quantize passes on the VALU butterfly kernels instead of the matrix cores (same
 *     bounds, another summation order); HQ_BOTH_NARROW=0 runs the two-sided X pass on 256-row
 *     half tiles at k <= 128; HQ_QUANT_REVERSE=0 keeps the forward tile order in the quantize
 *     passes of inputs of 128 MiB or more; HQ_COLS_REG=0 runs hq_fwht's LEFT butterflies at
 *     k = 16 on the LDS-staged kernel (another summation order); HQ_GEMM_NT=0 and
 *     HQ_FWHT_NT=0 store the products' and hq_fwht's VALU-kernel outputs without the
 *     non-temporal hint. HQ_SINGLE_SPIN and HQ_PAIR_SPIN bound the polls of the single-pass grid barrier
 *     and of the tile-pair exchange (0 forces their fallback paths).
 *     Rotations are computed in fp32 (the two-sided transform, rot BOTH, as fp32
 *     butterflies along the token axis over the fp32 values of V B). Quantization: s = absmax/Qp (fp32) or the given step,
 *     code = clamp(RNE(v * fp32(1/s)), -Qp, Qp), Qp = 127 (bits 8) or 7 (bits 4), or for E4M3
 *     codes the nearest E4M3 value of v * fp32(1/s) with s = absmax/448; a zero tensor gets
 *     s = 0 and all-zero codes. Integer GEMMs accumulate exactly in int32, FP8 GEMMs in fp32.
 *     Outputs are rounded to their dtype with round-to-nearest-even.
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HQ_ABI_VERSION 2

typedef enum {
  HQ_OK = 0,
  HQ_ERR_NULL = 1,      /* a required pointer is NULL */
  HQ_ERR_SHAPE = 2,     /* negative dim, or a rotated dim not divisible by k, or shape mismatch */
  HQ_ERR_K = 3,         /* k is not a power of two in [1, 256] */
  HQ_ERR_BITS = 4,      /* bits is not 4 or 8 (or not 8 for E4M3 codes) */
  HQ_ERR_DTYPE = 5,     /* unsupported dtype */
  HQ_ERR_MODE = 6,      /* bad rotation, scale mode, variant or code format */
  HQ_ERR_WORKSPACE = 7, /* workspace missing or smaller than hq_workspace_bytes() */
  HQ_ERR_MISMATCH = 8,  /* a saved qtensor does not match the call (k, bits, rot, format, shape) */
  HQ_ERR_DEVICE = 9,    /* no usable gfx950 device */
  HQ_ERR_LAUNCH = 10,   /* a kernel launch failed */
  HQ_ERR_ALIGN = 11     /* a device pointer or code row pitch is not 16-byte aligned */
} hq_status;

typedef enum { HQ_F32 = 0, HQ_F16 = 1, HQ_BF16 = 2 } hq_dtype;

/* Which block-diagonal rotation a tensor carries (INT4 page §3.3; HALO page, Approach):
 * RIGHT: V B (mixes columns within k-blocks);  LEFT: B V (mixes rows, the token axis);
 * BOTH: B V B;  NONE: V. */
typedef enum { HQ_ROT_NONE = 0, HQ_ROT_RIGHT = 1, HQ_ROT_LEFT = 2, HQ_ROT_BOTH = 3 } hq_rot;

/* ABSMAX: s = max|v| / Qp per tensor (HALO page, Approach / Limitations);
 * STEP: s is a given (learned) step (INT4 page §3.1). */
typedef enum { HQ_SCALE_ABSMAX = 0, HQ_SCALE_STEP = 1 } hq_scale_mode;

/* HALO0: no rotation (HALO page ablation baseline).
 * HQ:    X and W rotated on the right; dY quantized unrotated; backward reuses qW and qX
 *        (INT4 page §3.3, §4).
 * HALO2: HQ plus the left (token-axis) rotation of dY (HALO page, Approach). The weight
 *        gradient contracts over tokens against Q(B_N X B_C), written by the forward pass:
 *          Y  = (qX qW^T) sX sW / k
 *          dX = B_N (qG qW) B_C sG sW / k^2,   qG  = Q(B_N dY)
 *          dW = (qG^T qXt) B_C sG sXt / k^2,   qXt = Q(B_N X B_C) */
typedef enum { HQ_VARIANT_HALO0 = 0, HQ_VARIANT_HQ = 1, HQ_VARIANT_HALO2 = 2 } hq_variant;

/* Code format (HALO page: the three matmuls run in INT8 or in a floating-point format such as
 * FP8; an FP8 grid stands in where FP6 hardware is missing, Limitations):
 * INT:  integer codes on [-Qp, Qp] (bits 8: Qp = 127; bits 4: Qp = 7), integer GEMM with exact
 *       int32 accumulation;
 * E4M3: FP8 codes in the OCP E4M3 format (sign, 4-bit exponent with bias 7, 3-bit mantissa,
 *       subnormals, largest value 448, 0x7F/0xFF unused); bits must be 8. ABSMAX: s =
 *       absmax/448; a code is the E4M3 value nearest to v * fp32(1/s) (ties to even), saturating
 *       at +-448. The GEMM multiplies the codes on the matrix cores with fp32 accumulation.
 * E2M3, E3M2: FP6 codes (the same page's FP6 variants; it does not give the layout, so both OCP
 *       6-bit formats): E2M3 has a 2-bit exponent with bias 1 and a 3-bit mantissa, largest
 *       value 7.5; E3M2 a 3-bit exponent with bias 3 and a 2-bit mantissa, largest value 28;
 *       both have subnormals and no reserved patterns. bits must be 6. ABSMAX: s = absmax/7.5
 *       or absmax/28; a code is the FP6 value nearest to v * fp32(1/s) (ties to even),
 *       saturating. Every FP6 value is an E4M3 value, so a code is stored as the E4M3 byte of
 *       its value (one byte per code, like E4M3 codes) and the E4M3 GEMM multiplies them
 *       exactly: the FP8 product stands in for an FP6 one, as on the page. hq_rotated_stat's
 *       error sum and hq_select_hadamard_k take integer or E4M3 codes only. */
typedef enum { HQ_FMT_INT = 0, HQ_FMT_E4M3 = 1, HQ_FMT_E2M3 = 2, HQ_FMT_E3M2 = 3 } hq_format;

typedef struct {
  int32_t k;          /* Hadamard block size, power of two in [1, 256] (16..256 in practice) */
  int32_t bits;       /* 8 (INT8, Qp = 127; or E4M3), 4 (INT4 range [-7, 7], stored as int8), 6 (FP6) */
  int32_t scale_mode; /* hq_scale_mode */
  int32_t variant;    /* hq_variant */
  int32_t format;     /* hq_format */
} hq_config;

/* A quantized tensor: 8-bit codes (int8, or E4M3 bytes) of a rows x cols matrix plus its
 * device scale.
 * codes   : rows x cols, row pitch `ld` bytes (ld >= cols, ld % 16 == 0), or NULL.
 * codes_t : the transpose (cols x rows), row pitch `ld_t` bytes (ld_t >= rows,
 *           ld_t % 16 == 0), or NULL. It is the K-contiguous copy a backward product
 *           reads (INT4 page §A.6: the integer GEMM wants both operands K-contiguous).
 * Producers write zeros into the pitch padding, so consumers can read whole 16-byte rows.
 * rows, cols, k, bits, rot, format are written by the producer and checked by every
 * consumer. */
typedef struct {
  int8_t *codes;
  int8_t *codes_t;
  float *scale; /* one float on the device */
  int64_t rows, cols;
  int64_t ld, ld_t;
  int32_t k, bits, rot, format;
} hq_qtensor;

/* Version of this ABI (HQ_ABI_VERSION). */
int32_t hq_abi_version(void);

/* Static string for a status code (never NULL). */
const char *hq_status_string(int32_t status);

/* Row pitch (bytes) the library expects for a code matrix with `cols` columns: cols rounded
 * up to a multiple of 16. */
int64_t hq_code_pitch(int64_t cols);

/* Workspace bytes needed by any call of this library for a layer with these shapes and
 * this config (the maximum over hq_rotate_quantize on X, W, dY and the three products).
 * Returns 0 for invalid arguments. */
size_t hq_workspace_bytes(const hq_config *cfg, int64_t N, int64_t C, int64_t D);

/* Rotate -> tensor-wise scale -> quantize one rows x cols tensor (INT4 page §3.1, §3.3;
 * HALO page, Approach).
 *   src       rows x cols, row-major, dtype src_dtype (fp32/fp16/bf16)
 *   rot       rotation applied before quantization; rotated dims must be divisible by k
 *   step      STEP mode only: device pointer to one float (the step); ignored for ABSMAX
 *   out       host struct; out->codes and/or out->codes_t (at least one non-NULL) and
 *             out->scale are device buffers; the call fills rows, cols, k, bits, rot
 *   ws        workspace of ws_bytes (>= hq_workspace_bytes for a layer containing it)
 * Both code layouts carry the same rotation. For rot BOTH only out->codes_t is produced (the
 * transposed layout the weight-gradient product reads); out->codes must be NULL
 * (HQ_ERR_MODE otherwise) unless k == 1. */
hq_status hq_rotate_quantize(const void *src, int32_t src_dtype, int64_t rows, int64_t cols,
                             int32_t rot, const hq_config *cfg, const float *step,
                             hq_qtensor *out, void *ws, size_t ws_bytes, void *stream);

/* Forward Y = X W^T through HQ-MM (INT4 page §3.3, §A.6; HALO page, Approach).
 *   x, w      N x C and D x C, dtype in_dtype
 *   step_x, step_w, step_xt   STEP mode: device floats (step_xt: HALO2 only, may equal step_x)
 *   y         N x D output, dtype y_dtype
 *   save_x    required: receives Q(X B_C) (Q(X) under HALO0). codes is required (the forward
 *             operand); codes_t optional (the weight-gradient operand under HQ / HALO0)
 *   save_xt   HALO2 only, optional (NULL to skip): receives Q(B_N X B_C) in codes_t, for the
 *             weight gradient; N must then be divisible by k
 *   save_w    required: receives Q(W B_C); codes required, codes_t optional (dX operand)
 * The scales of the saved tensors are written on the device; backward calls reuse the codes
 * (INT4 page §4; HALO page, Approach). */
hq_status hq_linear_fwd(const void *x, const void *w, int32_t in_dtype, int64_t N, int64_t C,
                        int64_t D, const hq_config *cfg, const float *step_x,
                        const float *step_w, const float *step_xt, void *y, int32_t y_dtype,
                        hq_qtensor *save_x, hq_qtensor *save_xt, hq_qtensor *save_w,
                        void *ws, size_t ws_bytes, void *stream);

/* hq_linear_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, results and errors are those of hq_linear_fwd, whose kernels it runs; the
 * forward's scratch (absmax partials and grid-barrier words, under 20 KiB for any shape) lives
 * in a fixed device array of this library, one per GPU, held until the process ends. The first
 * call on a device looks the array's address up (no allocation); no call allocates or frees.
 * HQ_ERR_WORKSPACE if the forward ever needed more scratch than the array holds.
 * Calls that overlap on one GPU share that array and race: serialize them (one stream, or
 * events between streams). The array keeps the last call's contents; every call writes the
 * parts it reads before reading them. */
hq_status hq_linear_fwd_noalloc(const void *x, const void *w, int32_t in_dtype, int64_t N,
                                int64_t C, int64_t D, const hq_config *cfg,
                                const float *step_x, const float *step_w, const float *step_xt,
                                void *y, int32_t y_dtype, hq_qtensor *save_x,
                                hq_qtensor *save_xt, hq_qtensor *save_w, void *stream);

/* Input gradient dX = dY W (INT4 page §4; HALO page, Approach).
 *   dy        N x D, dtype dy_dtype
 *   step_g    STEP mode: device float
 *   saved_w   from hq_linear_fwd: needs codes_t (C x D) with rot RIGHT (NONE under HALO0)
 *   dx        N x C output, dtype dx_dtype
 *   save_g    required: receives Q(B_N dY) (HALO2) or Q(dY); codes required (this product's
 *             operand), codes_t optional (the weight-gradient operand). Under HALO2 N must
 *             be divisible by k. */
hq_status hq_linear_bwd_input(const void *dy, int32_t dy_dtype, int64_t N, int64_t C,
                              int64_t D, const hq_config *cfg, const float *step_g,
                              const hq_qtensor *saved_w, void *dx, int32_t dx_dtype,
                              hq_qtensor *save_g, void *ws, size_t ws_bytes, void *stream);

/* Weight gradient dW = dY^T X from saved codes only (INT4 page §4; HALO page, Approach).
 *   saved_g   from hq_linear_bwd_input: needs codes_t (D x N)
 *   saved_x   needs codes_t (C x N): save_xt of the forward under HALO2 (rot BOTH),
 *             save_x under HQ (rot RIGHT) or HALO0 (rot NONE)
 *   dw        D x C output, dtype dw_dtype */
hq_status hq_linear_bwd_weight(const hq_qtensor *saved_g, const hq_qtensor *saved_x,
                               int64_t N, int64_t C, int64_t D, const hq_config *cfg,
                               void *dw, int32_t dw_dtype, void *ws, size_t ws_bytes,
                               void *stream);

/* ---------------------------------------------------------------- batched products
 * Batched HQ-MM for the batched matmuls of attention (INT4 page §A.1: the same quantizers
 * apply to BMMs as to ordinary matrix multiplications). A batched operand is `batch` row-major
 * matrices stored one after another (e.g. heads x tokens x head_dim); batch b computes
 *   Y_b = X_b W_b^T (N x D),  dX_b = dY_b W_b (N x C),  dW_b = dY_b^T X_b (D x C)
 * with the rotations, variants and formats of the layer calls (e.g. scores S = Q K^T: X = Q,
 * W = K, C = head_dim; P V: X = P, W = V^T, C = key tokens). Each batched tensor is quantized
 * as one tensor: one scale for all batches, codes of the stacked (batch N) x C, (batch D) x C
 * and (batch N) x D matrices in the quantized-tensor structs, whose rows count every batch.
 * Right rotations act within rows and the token-axis blocks (N % k == 0 under HALO2) never
 * cross a batch, so the stacked codes are those of every batch. N and D must be multiples of
 * 16 when batch > 1 (HQ_ERR_SHAPE), batch at most 65535. Workspace: hq_bmm_workspace_bytes(cfg) bytes, for any
 * shape. Otherwise as hq_linear_fwd / hq_linear_bwd_input / hq_linear_bwd_weight. */
size_t hq_bmm_workspace_bytes(const hq_config *cfg);

hq_status hq_bmm_fwd(const void *x, const void *w, int32_t in_dtype, int64_t batch, int64_t N,
                     int64_t C, int64_t D, const hq_config *cfg, const float *step_x,
                     const float *step_w, const float *step_xt, void *y, int32_t y_dtype,
                     hq_qtensor *save_x, hq_qtensor *save_xt, hq_qtensor *save_w, void *ws,
                     size_t ws_bytes, void *stream);

hq_status hq_bmm_bwd_input(const void *dy, int32_t dy_dtype, int64_t batch, int64_t N,
                           int64_t C, int64_t D, const hq_config *cfg, const float *step_g,
                           const hq_qtensor *saved_w, void *dx, int32_t dx_dtype,
                           hq_qtensor *save_g, void *ws, size_t ws_bytes, void *stream);

hq_status hq_bmm_bwd_weight(const hq_qtensor *saved_g, const hq_qtensor *saved_x, int64_t batch,
                            int64_t N, int64_t C, int64_t D, const hq_config *cfg, void *dw,
                            int32_t dw_dtype, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- quantizer parameters
 * Statistics of a right-rotated tensor R = V B (rot RIGHT, blocks of cfg->k; rot NONE: R = V)
 * that set the quantizer parameters ("Training Transformers with 4-bit Integers", §3.1 learned
 * step, §A.3 step gradients by the chain rule from cheap elementwise residuals, §A.4 cold
 * start, §A.5 Hadamard size):
 *   HQ_STAT_ABS_SUM   sum |r|
 *   HQ_STAT_QERR      sum (r - s * value(code(r)))^2, code() the library's quantizer of cfg
 *                     (integer or E4M3), s = *scale
 *   HQ_STAT_LSQ_GRAD  sum (G B / k)_i * dv_hat_i/ds: the learned-step gradient of the loss with
 *                     respect to s, G = dL/dV (rows x cols, same dtype), straight-through
 *                     rounding: dv_hat/ds = code(r) - r/s inside the grid, +-Qp where clipped
 *                     (integer codes only; s must be > 0)
 * The terms are summed in fp64 (per-workgroup partials reduced in a fixed order) into *out
 * (one device double). The rotation is in fp32 as in hq_fwht. Workspace as hq_rotate_quantize. */
typedef enum { HQ_STAT_ABS_SUM = 0, HQ_STAT_QERR = 1, HQ_STAT_LSQ_GRAD = 2 } hq_stat_kind;

hq_status hq_rotated_stat(const void *src, const void *grad, int32_t dtype, int64_t rows,
                          int64_t cols, int32_t rot, const hq_config *cfg, int32_t stat,
                          const float *scale, double *out, void *ws, size_t ws_bytes,
                          void *stream);

/* Cold-start step of a tensor (INT4 page §A.4: before steps are learned a heuristic sets
 * them; the page does not give it, the library takes the learned-step initialisation):
 * *step = fp32(2 * mean|r| / sqrt(Qp)) over R = V B (or V), written on the device, ready as a
 * STEP-mode step. Integer codes only; HQ_ERR_SHAPE for an empty tensor. */
hq_status hq_cold_start_step(const void *src, int32_t dtype, int64_t rows, int64_t cols,
                             int32_t rot, const hq_config *cfg, float *step, void *ws,
                             size_t ws_bytes, void *stream);

/* Hadamard size selection (INT4 page §A.5): for each candidate k (powers of two dividing C,
 * at most HQ_MAX_K_CANDIDATES of them, host array), the quantization errors of X (N x C) and
 * W (D x C) with the tensor-wise absmax scale of X B_k and W B_k in cfg's format,
 * err = ||V - s Q(V B) B / k||_F^2 = sum (r - s q)^2 / k; *k_best (host) = the candidate with
 * the smallest err_X * err_W (ties: the earlier candidate); errors (host, 2 per candidate:
 * err_X, err_W) may be NULL. Runs on `stream` and WAITS for it (the choice is made on the
 * host): a setup-time call, not for graph capture. */
#define HQ_MAX_K_CANDIDATES 16
hq_status hq_select_hadamard_k(const void *x, const void *w, int32_t dtype, int64_t N,
                               int64_t C, int64_t D, const hq_config *cfg,
                               const int32_t *candidates, int32_t n_candidates, int32_t *k_best,
                               double *errors, void *ws, size_t ws_bytes, void *stream);

/* LSS-MM: the weight gradient of the INT4-range HQ layer from a leverage-score sample of the
 * tokens and a bit split of dY ("Training Transformers with 4-bit Integers": §4.2 bit splitting
 * and leverage score sampling; §A.2 the probability procedure; §A.6 INT8 data for the scores,
 * fused high/low quantization, zero padding of K after sampling; §B.2 the unbiased estimator):
 *   1. q8 = Q(dY) on the INT8 grid with the tensor-wise absmax step s8; the score of token i is
 *      l_i = ||q8_i|| * ||qX_i||, qX the forward's INT4 codes of X B_C (saved_x->codes);
 *   2. p = clamp-and-rescale probabilities with sum(p) = budget where possible: each round
 *      sets p_i = (budget' / sum_free(l)) l_i for the tokens not yet clamped (budget' = budget
 *      minus the clamped count), sets those above 1 to 1, and repeats until a round clamps
 *      none (zero scores: p = 0;
 *      budget >= the number of nonzero scores keeps every token with a nonzero score, the
 *      page's practical choice); sums in fp64, in a fixed order;
 *   3. token i is kept iff uniforms[i] < p_i (uniforms: N device floats in [0, 1), drawn by the
 *      caller); the K' kept tokens, in increasing order, are weighted by 1 / p_i;
 *   4. bit split of the kept weighted rows Gw = dY_i / p_i (fp64): s_hi = max|Gw| / 7,
 *      hi = Q_7(Gw / s_hi), s_lo = s_hi / 14, lo = Q_7((Gw - s_hi hi) / s_lo), codes
 *      14 hi + lo in [-105, 105];
 *   5. dW = ((14 hi + lo)^T qX_kept) [B_C] s_lo sX / k, one integer GEMM over the K' kept
 *      tokens (the page's two INT4 products, hi and lo, summed exactly in int32).
 * The codes of steps 1 and 4 follow the exact rule (round-to-nearest-even of the quotient,
 * ties decided exactly: fp32 products, with an fp64 fallback near ties). The steps are fp32:
 * s8 and s_hi are the correctly rounded quotients, s_lo = fp32(s_hi / 14).
 * cfg: format INT, bits 4, variant HQ (B_C of block size k) or HALO0 (no rotation); saved_x
 * as hq_linear_fwd writes it (row-major codes required, N x C). dy: N x D in dy_dtype.
 * Output dw: D x C in dw_dtype. Optional device outputs (NULL: kept in the workspace):
 * probs (N doubles, p), kept_idx (N int32, the first K' are the kept tokens), stats (one
 * hq_lss_stats). N <= 2^21 (int32 sums); workspace hq_lss_workspace_bytes(N, C, D).
 * The probability procedure runs on one workgroup: each round clamps at least one token, so
 * it ends after at most N rounds (a few for ordinary score spreads). */
typedef struct {
  int32_t kept; /* K', the number of sampled tokens */
  float s8;     /* step of the INT8 codes of dY behind the scores */
  float s_hi;   /* step of the high part of the bit split */
  float s_lo;   /* step of the low part (s_hi / 14) */
} hq_lss_stats;

size_t hq_lss_workspace_bytes(int64_t N, int64_t C, int64_t D);
hq_status hq_lss_bwd_weight(const void *dy, int32_t dy_dtype, const hq_qtensor *saved_x,
                            int64_t N, int64_t C, int64_t D, const hq_config *cfg, double budget,
                            const float *uniforms, void *dw, int32_t dw_dtype, double *probs,
                            int32_t *kept_idx, hq_lss_stats *stats, void *ws, size_t ws_bytes,
                            void *stream);

/* Standalone block-diagonal Walsh-Hadamard transform (unnormalized): dst = rotation of src
 * (INT4 page §3.3). rows x cols row-major; rotated dims divisible by k; rot != BOTH
 * for this entry point; src and dst must not overlap. Sums are formed in fp32 and rounded once
 * to dst_dtype (nearest even): exact whenever the fp32 sums are, else within the fp32
 * summation error of that. The implementation is hq_fwht_path's HQ_FWHT_AUTO choice: with
 * 16-bit src_dtype == dst_dtype, 16-byte aligned pointers and whole tiles (RIGHT: rows % 64
 * == 0, cols % 256 == 0; LEFT: rows % 256 == 0, cols % 64 == 0) the sums run on the matrix
 * cores for LEFT at k = 256, in another order than the VALU butterflies of the other cases. */
hq_status hq_fwht(const void *src, int32_t src_dtype, void *dst, int32_t dst_dtype,
                  int64_t rows, int64_t cols, int32_t rot, int32_t k, void *stream);

/* hq_fwht with the implementation named (for measuring one against the other; the results
 * agree to the fp32 summation order). path:
 *   HQ_FWHT_AUTO       what hq_fwht picks: the matrix cores where they cover the call and
 *                      were measured more than 5 % faster (LEFT at k = 256), the VALU
 *                      butterflies otherwise;
 *   HQ_FWHT_BUTTERFLY  the VALU butterflies (log2 k add/sub stages per element), any shape;
 *   HQ_FWHT_MATRIX     the matrix cores (a dense +-1 contraction in 16-bit MFMA, exact
 *                      products, fp32 sums); HQ_ERR_MODE unless the call has 16-bit
 *                      src_dtype == dst_dtype, 16-byte aligned pointers, k >= 16 and whole
 *                      tiles (RIGHT: rows % 64 == 0, cols % 256 == 0; LEFT: rows % 256 == 0,
 *                      cols % 64 == 0).
 * Other arguments and errors as hq_fwht. */
typedef enum { HQ_FWHT_AUTO = 0, HQ_FWHT_BUTTERFLY = 1, HQ_FWHT_MATRIX = 2 } hq_fwht_impl;

hq_status hq_fwht_path(const void *src, int32_t src_dtype, void *dst, int32_t dst_dtype,
                       int64_t rows, int64_t cols, int32_t rot, int32_t k, int32_t path,
                       void *stream);

/* Standalone integer GEMM with int32 accumulation (INT4 page §3.1, §A.6):
 *   c[m][n] = sum_k a[m][k] * b_t[n][k];  a: M x K (pitch lda), b_t: N x K (pitch ldb),
 *   c: M x N int32 (pitch N elements). lda, ldb multiples of 16 and >= K; bytes of a row
 *   between K and the next multiple of 16 must be zero. */
hq_status hq_gemm_i8_i32(const int8_t *a, int64_t lda, const int8_t *b_t, int64_t ldb,
                         int32_t *c, int64_t M, int64_t N, int64_t K, void *stream);

/* Standalone FP8 GEMM with fp32 accumulation (HALO page: FP8 matmuls; INT4 page §A.6 layouts):
 *   c[m][n] = sum_k a[m][k] * b_t[n][k] over E4M3 codes; a: M x K (pitch lda), b_t: N x K
 *   (pitch ldb), c: M x N fp32 (pitch N elements). lda, ldb multiples of 16 and >= K; bytes of a
 *   row between K and the next multiple of 16 must be zero. The products are exact; the sums
 *   are formed by the matrix cores in fp32 (not bit-reproducible against a sequential sum). */
hq_status hq_gemm_f8_f32(const uint8_t *a, int64_t lda, const uint8_t *b_t, int64_t ldb,
                         float *c, int64_t M, int64_t N, int64_t K, void *stream);

/* ---------------------------------------------------------------- instrumentation
 * Optional timing of the library's own kernel launches, for benchmarks (no compute).
 * hq_profile_start(mask) enables recording for the kernel kinds whose bit (1 << kind) is set:
 * each such launch is bracketed by two HIP events recorded on its own stream, together with
 * its algorithmic work in `units` (GEMM: 2*M*N*K integer ops; streaming kernels: bytes read
 * once plus bytes written once). hq_profile_stop waits for the recorded events, fills
 * stats[kind] for kind < n_stats (count, summed event time, summed units) and disables
 * recording. Process-wide state; not meant for concurrent use from several threads. */
typedef enum {
  HQ_KIND_GEMM = 0,         /* integer MFMA GEMM + dequantizing epilogue */
  HQ_KIND_ROT_ABSMAX = 1,   /* rotation + absmax partials */
  HQ_KIND_ROT_QUANT = 2,    /* rotation + quantization to codes */
  HQ_KIND_ROT_STORE = 3,    /* rotation to a floating-point output (inverse rotations, hq_fwht) */
  HQ_KIND_TRANSPOSE = 4,    /* int8 code transpose */
  HQ_KIND_MISC = 5,         /* scale writes, padding fills */
  HQ_KIND_COUNT = 6
} hq_kernel_kind;

typedef struct {
  int32_t kind;
  int32_t count;
  double total_ms;
  double units;
} hq_profile_stat;

hq_status hq_profile_start(uint32_t kind_mask);
hq_status hq_profile_stop(hq_profile_stat *stats, int32_t n_stats);

/* The launches recorded between the last hq_profile_start and hq_profile_stop, one record
 * each in launch order (kind, event time in ms, algorithmic units; `reserved` is 0). Copies
 * at most `cap` records into `out` (host memory; may be NULL when cap is 0) and returns how
 * many there are. Valid until the next hq_profile_start. */
typedef struct {
  int32_t kind;
  int32_t reserved;
  double ms;
  double units;
} hq_profile_record;

int32_t hq_profile_records(hq_profile_record *out, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
