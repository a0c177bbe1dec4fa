// hq_device.hpp — device helpers shared by the gfx950 kernels of libhq.
//
// Element formats, the in-register butterfly of the block-diagonal Walsh-Hadamard transform
// ("Training Transformers with 4-bit Integers", §3.3: H_k blocks), and the round-to-nearest
// quantizer onto the symmetric grid (same page, §3.1; HALO summary page, Limitations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// ----------------------------------------------------------------- element formats
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
  static constexpr bool is_bf16 = false;
  __device__ static inline float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static inline void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};

struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  static constexpr bool is_bf16 = false;
  __device__ static inline float from_bits(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
  __device__ static inline uint16_t to_bits(float v) {
    // v_cvt_f16_f32 rounds to nearest even in the default mode.
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
  __device__ static inline float load(const void* p, int64_t i) {
    return from_bits(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static inline void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = to_bits(v);
  }
  // Two values, each rounded to nearest even, packed low-first (one v_cvt_pk_f16_f32).
  __device__ static inline uint32_t pack2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, h2));
  }
};

struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  static constexpr bool is_bf16 = true;
  __device__ static inline float from_bits(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  __device__ static inline uint16_t to_bits(float v) {
    // round to nearest even on the dropped 16 bits (inputs are finite)
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
  __device__ static inline float load(const void* p, int64_t i) {
    return from_bits(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static inline void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = to_bits(v);
  }
  // Two values, each rounded to nearest even, packed low-first (one v_cvt_pk_bf16_f32).
  __device__ static inline uint32_t pack2(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, b2));
  }
};

// A compiler-only fence after a prefetch: the loads before it are issued before anything after
// it. A body that stores nothing (an absmax or a sum pass) would otherwise let the compiler sink
// the next item's loads down to their first use, which leaves one item's loads in flight and its
// latency exposed; the scheduling barrier also keeps the body's first instructions from moving
// above them. No instruction is emitted and no wait: the loads stay in flight across the fence.
__device__ inline void keep_issued() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16 consecutive elements as raw 16-byte chunks (two for 16-bit formats, four for fp32), so a
// prefetch holds no converted values; unpack16 converts them.
template <class T>
__device__ inline void load16_raw(const void* base, int64_t i0, uint4 (&q)[4]) {
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + i0 * T::bytes);
#pragma unroll
  for (int j = 0; j < T::bytes; ++j) q[j] = p[j];
}

template <class T>
__device__ inline void unpack16(const uint4 (&q)[4], float (&v)[16]) {
  if constexpr (T::bytes == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[4 * j + 0] = __uint_as_float(q[j].x); v[4 * j + 1] = __uint_as_float(q[j].y);
      v[4 * j + 2] = __uint_as_float(q[j].z); v[4 * j + 3] = __uint_as_float(q[j].w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * j + 2 * i + 0] = T::from_bits(static_cast<uint16_t>(w[i] & 0xFFFFu));
        v[8 * j + 2 * i + 1] = T::from_bits(static_cast<uint16_t>(w[i] >> 16));
      }
    }
  }
}

// Load 16 consecutive elements starting at element index i0 of a row whose valid length is
// n (elements >= n read as 0). `vec` says the row base and i0 are 16-byte aligned and the
// whole chunk is in bounds, so wide loads can be used.
template <class T>
__device__ inline void load16(const void* row, int64_t i0, int64_t n, bool vec, float (&v)[16]) {
  if (vec) {
    if constexpr (T::bytes == 4) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + i0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 f = p[q];
        v[4 * q + 0] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + i0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint4 u = p[q];
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * q + 2 * j + 0] = T::from_bits(static_cast<uint16_t>(w[j] & 0xFFFFu));
          v[8 * q + 2 * j + 1] = T::from_bits(static_cast<uint16_t>(w[j] >> 16));
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (i0 + j < n) ? T::load(row, i0 + j) : 0.0f;
  }
}

// u * alpha, or with PZ u * alpha + 0 (one fma): the same value except that a zero product
// is +0 whatever the signs of its factors.
template <bool PZ>
__device__ inline float scaled(float u, float alpha) {
  if constexpr (PZ) return __builtin_fmaf(u, alpha, 0.0f);
  return u * alpha;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte store, with the non-temporal (streaming) hint when NT.
template <bool NT>
__device__ inline void store16(char* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = v;
}

// Store u[0..N) * alpha as N consecutive elements starting at element `off` of `base`;
// only the first `nvalid` are written. Whole aligned runs use 16-byte stores. PZ: zero
// products are stored as +0 (for callers whose alpha carries a sign per lane). NT: the
// 16-byte stores carry the non-temporal hint (outputs no later kernel of the call reads).
template <class T, int N, bool PZ = false, bool NT = false>
__device__ inline void store_run(void* base, int64_t off, int64_t nvalid, const float (&u)[N],
                                 float alpha) {
  char* p = static_cast<char*>(base) + off * T::bytes;
  constexpr int PER16 = 16 / T::bytes;   // elements per 16-byte store
  if (nvalid >= N && N % PER16 == 0 && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
    for (int q = 0; q < N; q += PER16) {
      if constexpr (T::bytes == 4) {
        store16<NT>(p + 4 * q, u32x4{__float_as_uint(scaled<PZ>(u[q], alpha)),
                                     __float_as_uint(scaled<PZ>(u[q + 1], alpha)),
                                     __float_as_uint(scaled<PZ>(u[q + 2], alpha)),
                                     __float_as_uint(scaled<PZ>(u[q + 3], alpha))});
      } else {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = T::pack2(scaled<PZ>(u[q + 2 * j], alpha), scaled<PZ>(u[q + 2 * j + 1], alpha));
        store16<NT>(p + 2 * q, w);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < nvalid) T::store(base, off + q, scaled<PZ>(u[q], alpha));
  }
}

// ---------------------------------------------------------------- butterflies
// In-register stages of the unnormalized Walsh-Hadamard transform on N values that are N
// consecutive elements of a k-block: stride h pairs (i, i+h) -> (a+b, a-b), for h < min(K, N).
template <int K, int N>
__device__ inline void fwht_inreg(float (&v)[N]) {
#pragma unroll
  for (int h = 1; h < N && h < K; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Stages of fwht_inreg from stride H0 on (the smaller strides already applied).
template <int H0, int K, int N, class V>
__device__ inline void fwht_from(V (&v)[N]) {
#pragma unroll
  for (int h = H0; h < N && h < K; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & h) == 0) {
        V a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Value of lane (lane ^ m) within the wave.
__device__ inline float xor_lane(float x, int m) {
  return __shfl_xor(x, m, 64);
}

// One butterfly stage across lanes: lanes l and l^M hold the same positions of the two
// halves; the lane with the bit clear keeps a+b, the other keeps a-b (as fma(v, -1, p): the
// same single rounding). Strides inside a 16-lane row move through DPP on the VALU (quad
// permutes for 1 and 2; for 4 a row shift left into banks 0, 2 and right into banks 1, 3; for
// 8 a row rotate), wider ones through the LDS permute.
template <int M, int N>
__device__ inline void fwht_xlane_c(float (&v)[N], int lane) {
  const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int x = __float_as_int(v[i]);
    int p;
    if constexpr (M == 1) {
      p = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);            // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
      p = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);            // quad_perm 2,3,0,1
    } else if constexpr (M == 4) {
      p = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0x5, false);           // row_shl:4 -> l + 4
      p = __builtin_amdgcn_update_dpp(p, x, 0x114, 0xF, 0xA, false);     // row_shr:4 -> l - 4
    } else if constexpr (M == 8) {
      p = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);           // row_ror:8 -> l ^ 8
    } else {
      p = __shfl_xor(x, M, 64);
    }
    v[i] = __builtin_fmaf(v[i], sgn, __int_as_float(p));
  }
}

template <int N>
__device__ inline void fwht_xlane(float (&v)[N], int lane, int m) {
  switch (m) {   // m is a constant after unrolling: one case survives
    case 1: fwht_xlane_c<1, N>(v, lane); break;
    case 2: fwht_xlane_c<2, N>(v, lane); break;
    case 4: fwht_xlane_c<4, N>(v, lane); break;
    case 8: fwht_xlane_c<8, N>(v, lane); break;
    case 16: fwht_xlane_c<16, N>(v, lane); break;
    default: fwht_xlane_c<32, N>(v, lane); break;
  }
}

// Value of lane (lane ^ 1) / (lane ^ 2) within a quad, through DPP quad permutes.
__device__ inline float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ inline float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Butterfly stage across the lanes of a quad (m = 1 or 2): the lane with bit m clear keeps
// a + b, the other keeps a - b (a = lower lane's value, b = upper lane's value).
template <int N>
__device__ inline void quad_stage(float (&v)[N], int lane, int m) {
  const float sgn = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float p = (m == 1) ? quad_xor1(v[i]) : quad_xor2(v[i]);
    v[i] = __builtin_fmaf(v[i], sgn, p);   // lower: v + p, upper: p - v
  }
}

// ---------------------------------------------------------------- direct-to-LDS loads
constexpr int kBufferFlags = 0x00020000;   // raw untyped buffer, 32-bit records

// One 16-byte buffer load per lane straight into LDS: lane l's bytes land at lds + 16 l
// (the LDS base is wave-uniform and goes through M0).
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rs, int8_t* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}

// ---------------------------------------------------------------- reductions
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Block-wide max; every thread gets the result. `red` is __shared__ float[32].
__device__ inline float block_max(float x, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_max(x);
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < nw; ++w) r = fmaxf(r, red[w]);
  return r;
}

// ---------------------------------------------------------------- quantizer
// Scale of a tensor: the given step (STEP mode), or max(partials) / qmax (ABSMAX mode), qmax
// the grid bound (Qp, or the largest value of a float code format: 448, 7.5, 28).
// Every thread of the block returns the same (s, r = 1/s, or r = 0 when s == 0).
__device__ inline void tensor_scale(const float* partials, int nparts, const float* step,
                                    float qmax, float* red, float& s, float& r) {
  if (step != nullptr) {
    s = *step;
  } else {
    float a = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) a = fmaxf(a, partials[i]);
    a = block_max(a, red);
    s = a / qmax;   // correctly rounded fp32 division
  }
  r = (s > 0.0f) ? 1.0f / s : 0.0f;
}

// code = clamp(RNE(v * r), -qp, qp). The fma adds 1.5*2^23 to the exact product and rounds
// once, so the low mantissa bits hold RNE(v*r) in two's complement while |v*r| < 2^22; larger
// magnitudes still order correctly as float bit patterns, so the integer clamp saturates.
__device__ inline int quant_code(float v, float r, int qp) {
  const float magic = 12582912.0f;  // 1.5 * 2^23
  int bits = __float_as_int(__builtin_fmaf(v, r, magic));
  const int base = 0x4B400000;       // bit pattern of 1.5 * 2^23
  bits = min(max(bits, base - qp), base + qp);
  return bits - base;
}

// The same quantizer kept in the float domain: fma(v, r, 1.5*2^23) clamped to
// [1.5*2^23 - qp, 1.5*2^23 + qp] with med3; the low byte of the result's bit pattern is the
// code in two's complement. lo/hi are the two clamp bounds (exact floats).
__device__ inline uint32_t qbits(float v, float r, float lo, float hi) {
  return __float_as_uint(__builtin_amdgcn_fmed3f(__builtin_fmaf(v, r, 12582912.0f), lo, hi));
}
__device__ inline float qlo(int qp) { return 12582912.0f - static_cast<float>(qp); }
__device__ inline float qhi(int qp) { return 12582912.0f + static_cast<float>(qp); }

// Four codes (low bytes of qbits results) packed little-endian into one dword.
__device__ inline uint32_t qpack4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  return __builtin_amdgcn_perm(x1, x0, 0x0c0c0400u) | __builtin_amdgcn_perm(x3, x2, 0x04000c0cu);
}

// FP8 (OCP E4M3) codes: v * r clamped to [-448, 448] with med3, then the hardware conversion,
// which rounds to nearest even on the E4M3 grid (subnormals included) but turns values past
// 464 into the reserved code; the clamp makes it the saturating quantizer.
constexpr float kE4M3Max = 448.0f;

__device__ inline uint32_t e4m3_pack4(float v0, float v1, float v2, float v3, float r) {
  const float x0 = __builtin_amdgcn_fmed3f(v0 * r, -kE4M3Max, kE4M3Max);
  const float x1 = __builtin_amdgcn_fmed3f(v1 * r, -kE4M3Max, kE4M3Max);
  const float x2 = __builtin_amdgcn_fmed3f(v2 * r, -kE4M3Max, kE4M3Max);
  const float x3 = __builtin_amdgcn_fmed3f(v3 * r, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return static_cast<uint32_t>(w);
}

// FP6 codes (OCP E2M3: 3 mantissa bits, smallest normal 1, largest 7.5; E3M2: 2 mantissa bits,
// smallest normal 1/4, largest 28), kept as the E4M3 bytes of their values. x is already clamped
// to the format's range; its magnitude is rounded to the grid, ties to even: below the smallest
// normal a fixed step (1/8 or 1/16, the subnormals; rint is round to nearest even), above it the
// fp32 significand cut to the format's mantissa bits (add half an ulp minus one plus the kept
// lowest bit, then clear the dropped bits; a carry moves into the exponent as it should). The
// result is an E4M3 value, so the hardware conversion that follows is exact.
__device__ inline float fp6_round(float x, bool e3m2) {
  const float ax = fabsf(x);
  const float inv_step = e3m2 ? 16.0f : 8.0f, step = e3m2 ? 0.0625f : 0.125f;
  const float sub = __builtin_rintf(ax * inv_step) * step;
  const uint32_t drop = e3m2 ? 21u : 20u;   // 23 - mantissa bits
  uint32_t u = __float_as_uint(ax);
  u += ((1u << (drop - 1)) - 1u) + ((u >> drop) & 1u);
  u &= ~((1u << drop) - 1u);
  return __builtin_copysignf(ax < (e3m2 ? 0.25f : 1.0f) ? sub : __uint_as_float(u), x);
}

// Four float-format codes: v * r clamped to [-fmax, fmax], then, for the FP6 grids (grid 1 =
// E2M3, 2 = E3M2; 0 = E4M3 itself), rounded to the grid before the E4M3 conversion. grid and
// fmax are uniform.
__device__ inline uint32_t fcode_pack4(float v0, float v1, float v2, float v3, float r,
                                       float grid, float fmax) {
  float x0 = __builtin_amdgcn_fmed3f(v0 * r, -fmax, fmax);
  float x1 = __builtin_amdgcn_fmed3f(v1 * r, -fmax, fmax);
  float x2 = __builtin_amdgcn_fmed3f(v2 * r, -fmax, fmax);
  float x3 = __builtin_amdgcn_fmed3f(v3 * r, -fmax, fmax);
  if (grid != 0.0f) {
    const bool e3m2 = grid > 1.5f;
    x0 = fp6_round(x0, e3m2);
    x1 = fp6_round(x1, e3m2);
    x2 = fp6_round(x2, e3m2);
    x3 = fp6_round(x3, e3m2);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return static_cast<uint32_t>(w);
}

// Four codes of either kind packed little-endian into one dword: integer codes through qbits
// (lo, hi from qlo / qhi), or float-format codes (f8: lo = the grid, 0 E4M3, 1 E2M3, 2 E3M2;
// hi = the format's largest value; see float_bounds). f8 is uniform.
__device__ inline uint32_t quant4(float v0, float v1, float v2, float v3, float r, float lo,
                                  float hi, bool f8) {
  if (f8) return fcode_pack4(v0, v1, v2, v3, r, lo, hi);
  return qpack4(qbits(v0, r, lo, hi), qbits(v1, r, lo, hi), qbits(v2, r, lo, hi),
                qbits(v3, r, lo, hi));
}

// The (lo, hi) pair quant4 takes for float-format codes.
__device__ inline void float_bounds(int grid, float fmax, float& lo, float& hi) {
  lo = static_cast<float>(grid);
  hi = fmax;
}

// One code byte of either kind (two's complement integer, or a float-format code as above).
__device__ inline int quant_byte(float v, float r, int qp, bool f8, float grid, float fmax) {
  if (f8) return static_cast<int>(fcode_pack4(v, 0.0f, 0.0f, 0.0f, r, grid, fmax) & 0xFFu);
  return quant_code(v, r, qp);
}

// Pack 4 codes (already in [-127, 127]) into one little-endian dword.
__device__ inline uint32_t pack4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 0xFFu) | ((static_cast<uint32_t>(b) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(c) & 0xFFu) << 16) | ((static_cast<uint32_t>(d) & 0xFFu) << 24);
}

// v += sgn * v[lane ^ M] in one DPP instruction per value (quad permute, M = 1 or 2). With
// sgn = +1 on the lower lane of each pair and -1 on the upper, the lower lane gets a + b and
// the upper lane b - a, the negation of its butterfly output: each cross-lane stage flips the
// sign its upper lanes hold, and the caller folds that sign into the quantizer (a max of
// magnitudes is unaffected). The s_nop covers the VALU-write -> DPP-read hazard of whatever
// ran before the block.
template <int M>
__device__ inline void xstage8(float& v0, float& v1, float& v2, float& v3, float& v4, float& v5,
                               float& v6, float& v7, float sgn) {
  if constexpr (M == 1) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3), "+v"(v4), "+v"(v5), "+v"(v6), "+v"(v7)
        : "v"(sgn));
  } else {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3), "+v"(v4), "+v"(v5), "+v"(v6), "+v"(v7)
        : "v"(sgn));
  }
}

// Butterfly over lanes l and l ^ 4 (lane bit 2, inside a 16-lane row) in two DPP instructions
// per value: the lower lane of each pair (bit 2 clear, banks 0 and 2) takes a + b through a row
// shift left by four, the upper lane (banks 1 and 3) a - b through a row shift right by four.
// Each instruction writes only its banks of the new register and reads the old one, so the
// halves do not see each other's results. The s_nop covers the VALU-write -> DPP-read hazard
// of whatever wrote the inputs.
__device__ inline void xstage4_lane4(float (&v)[8]) {
  float r[8];
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %8, %8 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %0, %8, %8 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %9, %9 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %1, %9, %9 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %10, %10 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %2, %10, %10 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %11, %11 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %3, %11, %11 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %4, %12, %12 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %4, %12, %12 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %5, %13, %13 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %5, %13, %13 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %6, %14, %14 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %6, %14, %14 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %7, %15, %15 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_sub_f32_dpp %7, %15, %15 row_shr:4 row_mask:0xf bank_mask:0xa"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = r[i];
}

}  // namespace hq
