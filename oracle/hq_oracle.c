/*
 * hq_oracle.c — plain, slow CPU reference for the Hadamard-quantized linear-layer matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls this file;
 * only the test-suite, the smoke check and the CPU-baseline leg of the benchmark do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Every function is the plain definition of one step, written out with explicit loops:
 *   - H_k is the Sylvester Hadamard matrix built entry by entry (no fast transform);
 *   - rotations are dense sums against the explicit matrix;
 *   - the integer product is a triple loop accumulated in int64;
 *   - the output-side inverse rotations are exact int64 sums;
 *   - dequantization is done in double.
 *
 * Sources (cited by page title and section):
 *   [INT4]  "Training Transformers with 4-bit Integers" (paperlayer summary page)
 *           §3.1 learned step size quantizer, Q_N = Q_P = 7, INT32 product dequantized to FP16;
 *           §3.3 Hadamard quantization with block-diagonal H_k blocks, product preserved by
 *                inverse-transform cancellation;
 *           §4   backward reuses forward-quantized activations and weights;
 *           §A.6 HQ-MM stages: Hadamard multiplication, quantization, packing, INT GEMM,
 *                dequantization.
 *   [HALO]  "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs" (scime summary page)
 *           Approach: right-hand rotations on weights and activations in the forward pass,
 *                     left-hand rotation on output gradients in the backward pass (HALO-2),
 *                     tensor-wise quantization, reuse of quantized rotated tensors;
 *           Limitations: tensor-wise round-to-nearest quantization.
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - H is unnormalized (entries +-1, H*H^T = k*I) in natural Sylvester order,
 *     h(i,j) = (-1)^popcount(i & j); the 1/k factors go into the dequantization scalar.
 *   - Symmetric integer grid: codes in [-Qp, Qp], Qp = 127 (8 bit) or 7 (4-bit range).
 *   - Round to nearest, ties to even.
 *   - The code decision is taken in fp32, the precision the GPU kernel decides in:
 *       v32 = fp32(v) (v the rotated value), a32 = max |v32|, s = fp32(a32 / Qp),
 *       r = fp32(1 / s), q = clamp(RNE(v32 * r), -Qp, Qp) with the product exact.
 *     A zero tensor gets s = 0 and all-zero codes.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <fenv.h>

#define HQO_F32 0
#define HQO_F16 1
#define HQO_BF16 2

#define HQO_ROT_NONE 0
#define HQO_ROT_RIGHT 1
#define HQO_ROT_LEFT 2
#define HQO_ROT_BOTH 3

int hqo_version(void) { return 1; }

static int is_pow2_le256(int k) { return k >= 1 && k <= 256 && (k & (k - 1)) == 0; }

static int popcount_u32(uint32_t x) {
  int c = 0;
  while (x) { c += (int)(x & 1u); x >>= 1; }
  return c;
}

/* [INT4 §3.3] One H_k block, entry by entry: h(i,j) = +1 if popcount(i&j) is even, else -1.
 * Written row-major into H[k*k]. Returns 0, or -1 for an unsupported k. */
int hqo_hadamard(int k, int8_t *H) {
  if (!is_pow2_le256(k)) return -1;
  for (int i = 0; i < k; ++i)
    for (int j = 0; j < k; ++j)
      H[(int64_t)i * k + j] = (popcount_u32((uint32_t)(i & j)) & 1) ? -1 : 1;
  return 0;
}

/* Exact decode of fp32 / fp16 / bf16 bit patterns to double. */
static double decode_f16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);          /* (1024+m) * 2^(e-15-10) */
  return s ? -v : v;
}
static double decode_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}
int hqo_decode(const void *src, int dtype, int64_t n, double *dst) {
  if (dtype == HQO_F32) {
    const float *p = (const float *)src;
    for (int64_t i = 0; i < n; ++i) dst[i] = (double)p[i];
  } else if (dtype == HQO_F16) {
    const uint16_t *p = (const uint16_t *)src;
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_f16(p[i]);
  } else if (dtype == HQO_BF16) {
    const uint16_t *p = (const uint16_t *)src;
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_bf16(p[i]);
  } else {
    return -1;
  }
  return 0;
}

/* [INT4 §3.3, HALO Approach] Block-diagonal rotation with B = diag(H_k, ..., H_k), as dense sums
 * against the explicit matrix (long double accumulation):
 *   RIGHT: R = V * B,  R[i][b*k+j] = sum_t V[i][b*k+t] * h(t,j)    (mixes columns within blocks)
 *   LEFT : R = B * V,  R[b*k+i][j] = sum_t h(i,t) * V[b*k+t][j]    (mixes rows within blocks)
 *   BOTH : R = B * V * B (LEFT applied to the RIGHT result; both factors are the same H_k)
 *   NONE : copy.
 * V and R are rows x cols row-major; they must not alias. Returns 0, or -1 on bad arguments. */
int hqo_rotate(const double *V, int64_t rows, int64_t cols, int rot, int k, double *R) {
  if (!is_pow2_le256(k) || rows < 0 || cols < 0) return -1;
  if ((rot == HQO_ROT_RIGHT || rot == HQO_ROT_BOTH) && cols % k) return -1;
  if ((rot == HQO_ROT_LEFT || rot == HQO_ROT_BOTH) && rows % k) return -1;
  int8_t *H = (int8_t *)malloc((size_t)k * k);
  if (!H) return -1;
  hqo_hadamard(k, H);
  if (rot == HQO_ROT_NONE) {
    memcpy(R, V, sizeof(double) * (size_t)(rows * cols));
  } else if (rot == HQO_ROT_RIGHT) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t b = 0; b < cols / k; ++b)
        for (int j = 0; j < k; ++j) {
          long double acc = 0.0L;
          for (int t = 0; t < k; ++t)
            acc += (long double)V[i * cols + b * k + t] * (long double)H[t * k + j];
          R[i * cols + b * k + j] = (double)acc;
        }
  } else if (rot == HQO_ROT_LEFT) {
    /* Same sums as R[b*k+i][j] = sum_t h(i,t) V[b*k+t][j], each taken over t in ascending
     * order; the j loop runs innermost over a row accumulator so rows are read contiguously. */
#pragma omp parallel
    {
      long double *acc = (long double *)malloc(sizeof(long double) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static) collapse(2)
      for (int64_t b = 0; b < rows / k; ++b)
        for (int i = 0; i < k; ++i) {
          for (int64_t j = 0; j < cols; ++j) acc[j] = 0.0L;
          for (int t = 0; t < k; ++t) {
            const long double h = (long double)H[i * k + t];
            const double *vrow = V + (b * k + t) * cols;
            for (int64_t j = 0; j < cols; ++j) acc[j] += h * (long double)vrow[j];
          }
          for (int64_t j = 0; j < cols; ++j) R[(b * k + i) * cols + j] = (double)acc[j];
        }
      free(acc);
    }
  } else if (rot == HQO_ROT_BOTH) {
    double *T = (double *)malloc(sizeof(double) * (size_t)(rows * cols));
    if (!T) { free(H); return -1; }
    int rc = hqo_rotate(V, rows, cols, HQO_ROT_RIGHT, k, T);
    if (rc == 0) rc = hqo_rotate(T, rows, cols, HQO_ROT_LEFT, k, R);
    free(T);
    free(H);
    return rc;
  } else {
    free(H);
    return -1;
  }
  free(H);
  return 0;
}

/* [HALO Approach; INT4 §3.1] Tensor-wise scale, one per tensor.
 * ABSMAX: the value is rounded to fp32 first (the precision of the code decision), then
 *         a32 = max|v32| and s = fp32(a32 / Qp). Zero tensor -> 0.
 * The division is done in double and rounded once to fp32, which equals the correctly
 * rounded fp32 quotient of the two fp32 operands. */
float hqo_absmax_scale(const double *R, int64_t n, int qp) {
  float a32 = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float v32 = (float)R[i];
    float m = fabsf(v32);
    if (m > a32) a32 = m;
  }
  return (float)((double)a32 / (double)qp);
}

/* [INT4 §3.1; HALO Limitations] Round-to-nearest quantizer onto the symmetric grid [-Qp, Qp]:
 *   q = clamp(RNE(v32 * r), -Qp, Qp), r = fp32(1/s), product taken exactly (two fp32 values
 * multiply exactly in double). s == 0 gives all-zero codes. Returns 0. */
int hqo_quantize(const double *R, int64_t n, float scale, int qp, int8_t *q) {
  if (scale == 0.0f) {
    memset(q, 0, (size_t)n);
    return 0;
  }
  float r = (float)(1.0 / (double)scale);
  int old = fegetround();
  fesetround(FE_TONEAREST);
  for (int64_t i = 0; i < n; ++i) {
    float v32 = (float)R[i];
    double t = nearbyint((double)v32 * (double)r);
    if (t > qp) t = qp;
    if (t < -qp) t = -qp;
    q[i] = (int8_t)t;
  }
  fesetround(old);
  return 0;
}

/* [INT4 §3.1, §A.6] Integer matrix product with wide accumulation:
 *   C[m*N + n] = sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn]
 * Strides let one routine express the three products of a linear layer without copies.
 * Returns 0, or -1 when a sum leaves the int32 range the GPU accumulates in. */
int hqo_gemm_i8(const int8_t *A, int64_t sam, int64_t sak, const int8_t *B, int64_t sbk,
                int64_t sbn, int64_t M, int64_t N, int64_t K, int64_t *C) {
  int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int64_t acc = 0;
      for (int64_t k = 0; k < K; ++k)
        acc += (int64_t)A[m * sam + k * sak] * (int64_t)B[k * sbk + n * sbn];
      if (acc > INT32_MAX || acc < INT32_MIN) overflow = 1;
      C[m * N + n] = acc;
    }
  return overflow ? -1 : 0;
}

/* [INT4 §3.3] Inverse rotation of an integer product, exact in int64 (the same explicit H;
 * H^-1 = H/k and the 1/k goes to the dequantization scalar). Same index maps as hqo_rotate. */
int hqo_rotate_i64(const int64_t *T, int64_t rows, int64_t cols, int rot, int k, int64_t *R) {
  if (!is_pow2_le256(k) || rows < 0 || cols < 0) return -1;
  if ((rot == HQO_ROT_RIGHT || rot == HQO_ROT_BOTH) && cols % k) return -1;
  if ((rot == HQO_ROT_LEFT || rot == HQO_ROT_BOTH) && rows % k) return -1;
  int8_t *H = (int8_t *)malloc((size_t)k * k);
  if (!H) return -1;
  hqo_hadamard(k, H);
  if (rot == HQO_ROT_NONE) {
    memcpy(R, T, sizeof(int64_t) * (size_t)(rows * cols));
  } else if (rot == HQO_ROT_RIGHT) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t b = 0; b < cols / k; ++b)
        for (int j = 0; j < k; ++j) {
          int64_t acc = 0;
          for (int t = 0; t < k; ++t) acc += T[i * cols + b * k + t] * (int64_t)H[t * k + j];
          R[i * cols + b * k + j] = acc;
        }
  } else if (rot == HQO_ROT_LEFT) {
    /* R[b*k+i][j] = sum_t h(i,t) T[b*k+t][j] (exact integers; rows read contiguously) */
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t b = 0; b < rows / k; ++b)
      for (int i = 0; i < k; ++i) {
        int64_t *out = R + (b * k + i) * cols;
        for (int64_t j = 0; j < cols; ++j) out[j] = 0;
        for (int t = 0; t < k; ++t) {
          const int64_t h = (int64_t)H[i * k + t];
          const int64_t *trow = T + (b * k + t) * cols;
          for (int64_t j = 0; j < cols; ++j) out[j] += h * trow[j];
        }
      }
  } else if (rot == HQO_ROT_BOTH) {
    int64_t *U = (int64_t *)malloc(sizeof(int64_t) * (size_t)(rows * cols));
    if (!U) { free(H); return -1; }
    int rc = hqo_rotate_i64(T, rows, cols, HQO_ROT_RIGHT, k, U);
    if (rc == 0) rc = hqo_rotate_i64(U, rows, cols, HQO_ROT_LEFT, k, R);
    free(U);
    free(H);
    return rc;
  } else {
    free(H);
    return -1;
  }
  free(H);
  return 0;
}

/* [INT4 §3.1] Dequantization: out = T * s_a * s_b / k^e in double. */
void hqo_dequant(const int64_t *T, int64_t n, float s_a, float s_b, int k_pow_e, double *out) {
  double alpha = (double)s_a * (double)s_b / (double)k_pow_e;
  for (int64_t i = 0; i < n; ++i) out[i] = (double)T[i] * alpha;
}

/* Round double values to an output dtype with round-to-nearest-even, written as raw bits
 * (float for fp32; uint16 patterns for fp16 / bf16). Used to compare against a GPU output of
 * the same dtype. Values are finite and within range by construction. */
static uint16_t round_f16(double v) {
  /* fp16: 11 significant bits; subnormals are multiples of 2^-24. */
  uint16_t sign = 0;
  if (v < 0 || (v == 0 && signbit(v))) { sign = 0x8000; v = -v; }
  if (v == 0) return sign;
  if (v >= 65520.0) return sign | 0x7c00; /* overflow to inf */
  int e;
  frexp(v, &e); /* v = f * 2^e, f in [0.5,1) -> leading bit weight 2^(e-1) */
  int exp_unb = e - 1;
  if (exp_unb < -14) exp_unb = -14; /* subnormal range: quantum 2^-24 */
  double quantum = ldexp(1.0, exp_unb - 10);
  double m = nearbyint(v / quantum); /* RNE (FE_TONEAREST set by caller) */
  double r = m * quantum;
  /* re-encode */
  if (r == 0) return sign;
  int e2;
  frexp(r, &e2);
  int eb = e2 - 1;
  if (eb < -14) { /* subnormal */
    return sign | (uint16_t)(r / ldexp(1.0, -24));
  }
  if (eb > 15) return sign | 0x7c00;
  uint16_t mant = (uint16_t)(r / ldexp(1.0, eb - 10) - 1024.0);
  return sign | (uint16_t)((eb + 15) << 10) | mant;
}
static uint16_t round_bf16(double v) {
  /* bf16: 8 significant bits, exponent range of fp32. Round in one step from double. */
  uint16_t sign = 0;
  if (v < 0 || (v == 0 && signbit(v))) { sign = 0x8000; v = -v; }
  if (v == 0) return sign;
  int e;
  frexp(v, &e);
  int exp_unb = e - 1;
  if (exp_unb < -126) exp_unb = -126; /* subnormal quantum 2^-133 */
  double quantum = ldexp(1.0, exp_unb - 7);
  double r = nearbyint(v / quantum) * quantum;
  float f = (float)r; /* exact: r has <= 8 significant bits within fp32 range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}
int hqo_round(const double *src, int64_t n, int dtype, void *dst) {
  int old = fegetround();
  fesetround(FE_TONEAREST);
  if (dtype == HQO_F32) {
    float *p = (float *)dst;
    for (int64_t i = 0; i < n; ++i) p[i] = (float)src[i];
  } else if (dtype == HQO_F16) {
    uint16_t *p = (uint16_t *)dst;
    for (int64_t i = 0; i < n; ++i) p[i] = round_f16(src[i]);
  } else if (dtype == HQO_BF16) {
    uint16_t *p = (uint16_t *)dst;
    for (int64_t i = 0; i < n; ++i) p[i] = round_bf16(src[i]);
  } else {
    fesetround(old);
    return -1;
  }
  fesetround(old);
  return 0;
}
