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
 *   - The scale and the code are the plain definitions, taken exactly from the rotated value R
 *     (summed in long double, exact for the 16-bit inputs used here):
 *       a = max |R|,  s = a / Qp rounded once to fp32 (the scale is stored as one fp32),
 *       q = clamp(RNE(R / s), -Qp, Qp), the quotient compared exactly against the midpoints
 *       (q +- 1/2) * s, so no intermediate rounding can move a code.
 *     A zero tensor gets s = 0 and all-zero codes.
 *   - FP8 codes (HALO page: the variants that run all three matmuls in FP8/FP6; an FP8 grid is
 *     used where FP6 hardware is missing, Limitations) are the OCP E4M3 format: sign, 4-bit
 *     exponent with bias 7, 3-bit mantissa, subnormals m * 2^-9, largest finite value 448, and
 *     the code 0x7F / 0xFF reserved (not a number). The tensor-wise scale is s = max|R| / 448 and
 *     a code is the E4M3 value nearest to R / s, ties to the even mantissa, saturating at
 *     +-448; a value that rounds to zero keeps its sign bit. Every E4M3 value is an integer
 *     multiple of 2^-9, so products of two codes are exact integers in units of 2^-18 and the
 *     integer product below accumulates them exactly in int64.
 *   - FP6 codes (the same page's FP6 variants; the layout is not given) are either OCP 6-bit
 *     format, E2M3 (largest 7.5) or E3M2 (largest 28): s = max|R| / largest value, the
 *     nearest FP6 value, ties to the even mantissa, saturating. Both grids lie inside E4M3, so
 *     an FP6 code is kept as the E4M3 byte of its value and the FP8 product serves.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HQO_F32 0
#define HQO_F16 1
#define HQO_BF16 2

#define HQO_ROT_NONE 0
#define HQO_ROT_RIGHT 1
#define HQO_ROT_LEFT 2
#define HQO_ROT_BOTH 3

int hqo_version(void) { return 1; }

/* Threads the OpenMP loops of this library run on (1 when built without OpenMP). */
int hqo_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

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

static int f32_odd(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (int)(u & 1u);
}

/* Correctly rounded fp32 value of the exact quotient a / d (a >= 0 finite, d > 0 with at most
 * 7 significant bits: 127, 7, 448, 7.5 or 28). Start from the double quotient rounded to fp32, then move to a neighbour while the
 * exact quotient lies beyond the midpoint towards it (on the midpoint: to the even
 * significand). A midpoint of two fp32 values has 25 significant bits, so midpoint * d is
 * exact in double and every comparison is exact. */
static float div_to_f32(double a, double d) {
  float f = (float)(a / (double)d);
  for (;;) {
    const float up = nextafterf(f, INFINITY), dn = nextafterf(f, 0.0f);
    const double hi = ((double)f + (double)up) * 0.5 * d;
    const double lo = ((double)f + (double)dn) * 0.5 * d;
    if (a > hi || (a == hi && f32_odd(f))) { f = up; continue; }
    if (f > 0.0f && (a < lo || (a == lo && f32_odd(f)))) { f = dn; continue; }
    return f;
  }
}

/* [HALO Approach; INT4 §3.1] Tensor-wise scale, one per tensor: a = max |R| over the exact
 * rotated values, s = a / Qp correctly rounded to fp32. Zero tensor -> 0. */
float hqo_absmax_scale(const double *R, int64_t n, int qp) {
  double a = 0.0;
  for (int64_t i = 0; i < n; ++i)
    if (fabs(R[i]) > a) a = fabs(R[i]);
  return div_to_f32(a, (double)qp);
}

/* The same with a grid bound that need not be an integer (7.5, the largest E2M3 value): it has
 * at most 4 significant bits, so midpoint * d stays exact in double. */
float hqo_absmax_scale_d(const double *R, int64_t n, double qmax) {
  double a = 0.0;
  for (int64_t i = 0; i < n; ++i)
    if (fabs(R[i]) > a) a = fabs(R[i]);
  return div_to_f32(a, qmax);
}

/* [INT4 §3.1; HALO Limitations] Round-to-nearest quantizer onto the symmetric grid [-Qp, Qp]:
 *   q = clamp(RNE(R / s), -Qp, Qp).
 * The quotient is never rounded: for |R| < (Qp + 1) s the code q is found by exact
 * comparisons of R against the midpoints (q - 1/2) s and (q + 1/2) s (each a product of a
 * short dyadic and an fp32 value, exact in double); a value on a midpoint goes to the even
 * neighbour. Beyond that range the clamp decides. s == 0 gives all-zero codes. Returns 0. */
int hqo_quantize(const double *R, int64_t n, float scale, int qp, int8_t *q) {
  if (scale == 0.0f) {
    memset(q, 0, (size_t)n);
    return 0;
  }
  const double s = (double)scale;
  const double lim = ((double)qp + 1.0) * s;
  for (int64_t i = 0; i < n; ++i) {
    const double v = R[i];
    int c;
    if (v >= lim) {
      c = qp;
    } else if (v <= -lim) {
      c = -qp;
    } else {
      c = (int)(v / s);                                /* a start near the answer */
      while (v > ((double)c + 0.5) * s) ++c;           /* now v <= (c + 1/2) s */
      while (v < ((double)c - 0.5) * s) --c;           /* now (c - 1/2) s <= v <= (c + 1/2) s */
      if (v == ((double)c + 0.5) * s && (c & 1)) ++c;  /* midpoint: the even neighbour */
      if (v == ((double)c - 0.5) * s && (c & 1)) --c;
      if (c > qp) c = qp;
      if (c < -qp) c = -qp;
    }
    q[i] = (int8_t)c;
  }
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

/* ---------------------------------------------------------------- FP8 (E4M3) codes
 * Value of an E4M3 code in units of 2^-9 (an integer): subnormal (exponent field 0) m, normal
 * (8 + m) * 2^(e - 1). Returns 0 for the two reserved codes, which the quantizer never writes. */
static int64_t e4m3_units(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return 0;
  const int64_t mag = (e == 0) ? m : (int64_t)(8 + m) << (e - 1);
  return (c & 0x80) ? -mag : mag;
}

/* Decode E4M3 codes to double (exact). */
void hqo_decode_e4m3(const uint8_t *q, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ldexp((double)e4m3_units(q[i]), -9);
}

/* [HALO summary page, Key results / Limitations: FP8 as the lower-precision grid]
 * q = the E4M3 code nearest to R / s (ties to the even mantissa, saturating at +-448).
 * Magnitude codes 0..126 are the non-negative grid in increasing order (code 126 = 448). The
 * code is found by exact comparisons of |R| against g(c) * s and against the midpoints
 * (g(c) + g(c + 1)) / 2 * s, where g(c) has at most 4 significant bits, so every product with
 * the fp32 step is exact in double. s == 0 gives all-zero codes. Returns 0. */
int hqo_quantize_e4m3(const double *R, int64_t n, float scale, uint8_t *q) {
  if (scale == 0.0f) {
    memset(q, 0, (size_t)n);
    return 0;
  }
  const double s = (double)scale;
  for (int64_t i = 0; i < n; ++i) {
    const double a = fabs(R[i]);
    int c = 0;
    /* largest magnitude code whose value times s is <= |R| (binary search over 0..126) */
    int lo = 0, hi = 126;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (ldexp((double)e4m3_units((uint8_t)mid), -9) * s <= a) lo = mid;
      else hi = mid - 1;
    }
    c = lo;
    if (c < 126) {
      const double g0 = ldexp((double)e4m3_units((uint8_t)c), -9);
      const double g1 = ldexp((double)e4m3_units((uint8_t)(c + 1)), -9);
      const double midv = (g0 + g1) * 0.5 * s;
      if (a > midv || (a == midv && (c & 1))) ++c;   /* nearest; a tie goes to the even code */
    }
    q[i] = (uint8_t)(c | (signbit(R[i]) ? 0x80 : 0));
  }
  return 0;
}

/* ---------------------------------------------------------------- FP6 codes (E2M3, E3M2)
 * [HALO summary page, Key results (the FP6 variants of the matmuls) and Limitations (tensor-wise
 * round-to-nearest; FP8 matmuls stood in for FP6 on hardware without FP6)]. The pages do not fix
 * the layout; both OCP 6-bit formats are provided: sign, E exponent bits with bias
 * 2^(E-1) - 1, M mantissa bits, subnormals, every pattern finite. E2M3 (E = 2, M = 3) spans
 * [-7.5, 7.5] in steps of 1/8 near zero; E3M2 (E = 3, M = 2) spans [-28, 28] in steps of 1/16
 * near zero. Magnitude ordinal c = (e << M) | m, increasing in value: m 2^(1 - bias - M) for
 * e = 0, (2^M + m) 2^(e - bias - M) otherwise. Every FP6 value of either format is an E4M3
 * value (at most 3 significant bits, exponents inside E4M3's range), so a code is stored as
 * the E4M3 byte of its value, and the FP8 product, decode and dequantization apply unchanged.
 * fmt: 2 = E2M3, 3 = E3M2 (the library's format numbers). */
static int fp6_layout(int fmt, int *E, int *M) {
  if (fmt == 2) { *E = 2; *M = 3; return 0; }
  if (fmt == 3) { *E = 3; *M = 2; return 0; }
  return -1;
}

/* Value of FP6 magnitude ordinal c in units of 2^-9 (an integer for both formats). */
static int64_t fp6_units(int E, int M, int c) {
  const int bias = (1 << (E - 1)) - 1, e = c >> M, m = c & ((1 << M) - 1);
  const int64_t mant = (e == 0) ? m : (int64_t)((1 << M) + m);
  const int ex = (e == 0 ? 1 : e) - bias - M + 9;   /* >= 5 for both formats */
  return mant << ex;
}

/* E4M3 byte of a non-negative value given in units of 2^-9 that lies on the E4M3 grid. */
static int e4m3_code_of(int64_t units) {
  int lo = 0, hi = 126;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (e4m3_units((uint8_t)mid) < units) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

/* The largest FP6 value of the format (the grid bound the tensor-wise scale maps max |R| to). */
double hqo_fp6_max(int fmt) {
  int E, M;
  if (fp6_layout(fmt, &E, &M)) return -1.0;
  return ldexp((double)fp6_units(E, M, (1 << (E + M)) - 1), -9);
}

/* q = the FP6 value nearest to R / s, ties to the even magnitude ordinal (the even mantissa),
 * saturating at the largest value, stored as its E4M3 byte; a value that rounds to zero keeps
 * its sign bit, as for E4M3 codes. The ordinal is found by exact comparisons of |R| against
 * g(c) s and the midpoints (g(c) + g(c + 1)) / 2 s, each exact in double. s == 0 gives all-zero
 * codes. Returns -1 for an unknown format, else 0. */
int hqo_quantize_fp6(const double *R, int64_t n, float scale, int fmt, uint8_t *q) {
  int E, M;
  if (fp6_layout(fmt, &E, &M)) return -1;
  if (scale == 0.0f) {
    memset(q, 0, (size_t)n);
    return 0;
  }
  const int cmax = (1 << (E + M)) - 1;
  const double s = (double)scale;
  for (int64_t i = 0; i < n; ++i) {
    const double a = fabs(R[i]);
    int lo = 0, hi = cmax;   /* largest ordinal whose value times s is <= |R| */
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (ldexp((double)fp6_units(E, M, mid), -9) * s <= a) lo = mid;
      else hi = mid - 1;
    }
    int c = lo;
    if (c < cmax) {
      const double g0 = ldexp((double)fp6_units(E, M, c), -9);
      const double g1 = ldexp((double)fp6_units(E, M, c + 1), -9);
      const double midv = (g0 + g1) * 0.5 * s;
      if (a > midv || (a == midv && (c & 1))) ++c;   /* nearest; a tie goes to the even ordinal */
    }
    q[i] = (uint8_t)(e4m3_code_of(fp6_units(E, M, c)) | (signbit(R[i]) ? 0x80 : 0));
  }
  return 0;
}

/* [INT4 §3.1, §A.6 with FP8 codes] Exact product of two E4M3 code matrices, in units of 2^-18:
 *   C[m*N + n] = sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn] (code values times 2^9 each).
 * |A B| <= 448^2 2^18 K stays far inside int64 for every K used here. Returns 0. */
int hqo_gemm_f8(const uint8_t *A, int64_t sam, int64_t sak, const uint8_t *B, int64_t sbk,
                int64_t sbn, int64_t M, int64_t N, int64_t K, int64_t *C) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int64_t acc = 0;
      for (int64_t k = 0; k < K; ++k)
        acc += e4m3_units(A[m * sam + k * sak]) * e4m3_units(B[k * sbk + n * sbn]);
      C[m * N + n] = acc;
    }
  return 0;
}

/* [INT4 §3.3] Inverse rotation of an integer product, exact in int64 (the same explicit H;
 * H^-1 = H/k and the 1/k goes to the dequantization scalar). Same index maps as hqo_rotate.
 * Returns -1 if a sum would leave the int64 range. */
int hqo_rotate_i64(const int64_t *T, int64_t rows, int64_t cols, int rot, int k, int64_t *R) {
  if (!is_pow2_le256(k) || rows < 0 || cols < 0) return -1;
  if ((rot == HQO_ROT_RIGHT || rot == HQO_ROT_BOTH) && cols % k) return -1;
  if ((rot == HQO_ROT_LEFT || rot == HQO_ROT_BOTH) && rows % k) return -1;
  int8_t *H = (int8_t *)malloc((size_t)k * k);
  if (!H) return -1;
  hqo_hadamard(k, H);
  int overflow = 0;   /* a sum left the int64 range (never for the products used here) */
  if (rot == HQO_ROT_NONE) {
    memcpy(R, T, sizeof(int64_t) * (size_t)(rows * cols));
  } else if (rot == HQO_ROT_RIGHT) {
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t b = 0; b < cols / k; ++b)
        for (int j = 0; j < k; ++j) {
          int64_t acc = 0;
          for (int t = 0; t < k; ++t)
            if (__builtin_add_overflow(acc, T[i * cols + b * k + t] * (int64_t)H[t * k + j], &acc))
              overflow = 1;
          R[i * cols + b * k + j] = acc;
        }
  } else if (rot == HQO_ROT_LEFT) {
    /* R[b*k+i][j] = sum_t h(i,t) T[b*k+t][j] (exact integers; rows read contiguously) */
#pragma omp parallel for schedule(static) collapse(2) reduction(| : overflow)
    for (int64_t b = 0; b < rows / k; ++b)
      for (int i = 0; i < k; ++i) {
        int64_t *out = R + (b * k + i) * cols;
        for (int64_t j = 0; j < cols; ++j) out[j] = 0;
        for (int t = 0; t < k; ++t) {
          const int64_t h = (int64_t)H[i * k + t];
          const int64_t *trow = T + (b * k + t) * cols;
          for (int64_t j = 0; j < cols; ++j)
            if (__builtin_add_overflow(out[j], h * trow[j], &out[j])) overflow = 1;
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
  return overflow ? -1 : 0;
}

/* [INT4 §3.1] Dequantization: out = T * s_a * s_b / div in double, div = k^e (a power of two;
 * for FP8 products also times 2^18, the unit of the exact FP8 sums). */
void hqo_dequant(const int64_t *T, int64_t n, float s_a, float s_b, double div, double *out) {
  double alpha = (double)s_a * (double)s_b / div;
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
