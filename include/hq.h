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
 *     default stream). Scales stay on the device; no call synchronizes with the host.
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
 *     Rotations are computed in fp32, except the token-axis rotation of the two-sided
 *     transform (rot BOTH), which sums the fp32 values of V B exactly in fp64 and rounds the
 *     result to fp32 once. Quantization: s = absmax/Qp (fp32) or the given step,
 *     code = clamp(RNE(v * fp32(1/s)), -Qp, Qp), Qp = 127 (bits 8) or 7 (bits 4); a zero
 *     tensor gets s = 0 and all-zero codes. Integer GEMMs accumulate exactly in int32.
 *     Outputs are rounded to their dtype with round-to-nearest-even.
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HQ_ABI_VERSION 1

typedef enum {
  HQ_OK = 0,
  HQ_ERR_NULL = 1,      /* a required pointer is NULL */
  HQ_ERR_SHAPE = 2,     /* negative dim, or a rotated dim not divisible by k, or shape mismatch */
  HQ_ERR_K = 3,         /* k is not a power of two in [1, 256] */
  HQ_ERR_BITS = 4,      /* bits is not 4 or 8 */
  HQ_ERR_DTYPE = 5,     /* unsupported dtype */
  HQ_ERR_MODE = 6,      /* bad rotation, scale mode or variant */
  HQ_ERR_WORKSPACE = 7, /* workspace missing or smaller than hq_workspace_bytes() */
  HQ_ERR_MISMATCH = 8,  /* a saved qtensor does not match the call (k, bits, rot, shape) */
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

typedef struct {
  int32_t k;          /* Hadamard block size, power of two in [1, 256] (16..256 in practice) */
  int32_t bits;       /* 8 (INT8, Qp = 127) or 4 (INT4 range [-7, 7], stored as int8) */
  int32_t scale_mode; /* hq_scale_mode */
  int32_t variant;    /* hq_variant */
} hq_config;

/* A quantized tensor: int8 codes of a rows x cols matrix plus its device scale.
 * codes   : rows x cols, row pitch `ld` bytes (ld >= cols, ld % 16 == 0), or NULL.
 * codes_t : the transpose (cols x rows), row pitch `ld_t` bytes (ld_t >= rows,
 *           ld_t % 16 == 0), or NULL. It is the K-contiguous copy a backward product
 *           reads (INT4 page §A.6: the integer GEMM wants both operands K-contiguous).
 * Producers write zeros into the pitch padding, so consumers can read whole 16-byte rows.
 * rows, cols, k, bits, rot are written by the producer and checked by every consumer. */
typedef struct {
  int8_t *codes;
  int8_t *codes_t;
  float *scale; /* one float on the device */
  int64_t rows, cols;
  int64_t ld, ld_t;
  int32_t k, bits, rot, reserved;
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

/* Standalone block-diagonal Walsh-Hadamard transform (unnormalized): dst = rotation of src
 * (INT4 page §3.3). rows x cols row-major; rotated dims divisible by k; rot != BOTH
 * for this entry point; src and dst must not overlap. Sums are formed in fp32 and rounded once
 * to dst_dtype (nearest even): exact whenever the fp32 sums are, else within the fp32
 * summation error of that. With 16-bit src_dtype == dst_dtype, 16-byte aligned pointers and
 * whole tiles (RIGHT: rows % 64 == 0, cols % 256 == 0, k >= 128; LEFT: rows % 256 == 0,
 * cols % 64 == 0, k >= 16) the sums run on the matrix cores, in another order than the VALU
 * butterflies of the other cases. */
hq_status hq_fwht(const void *src, int32_t src_dtype, void *dst, int32_t dst_dtype,
                  int64_t rows, int64_t cols, int32_t rot, int32_t k, void *stream);

/* Standalone integer GEMM with int32 accumulation (INT4 page §3.1, §A.6):
 *   c[m][n] = sum_k a[m][k] * b_t[n][k];  a: M x K (pitch lda), b_t: N x K (pitch ldb),
 *   c: M x N int32 (pitch N elements). lda, ldb multiples of 16 and >= K; bytes of a row
 *   between K and the next multiple of 16 must be zero. */
hq_status hq_gemm_i8_i32(const int8_t *a, int64_t lda, const int8_t *b_t, int64_t ldb,
                         int32_t *c, int64_t M, int64_t N, int64_t K, void *stream);

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

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
