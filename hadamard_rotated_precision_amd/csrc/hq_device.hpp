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

// Store u[0..N) * alpha as N consecutive elements starting at element `off` of `base`;
// only the first `nvalid` are written. Whole aligned runs use 16-byte stores.
template <class T, int N>
__device__ inline void store_run(void* base, int64_t off, int64_t nvalid, const float (&u)[N],
                                 float alpha) {
  char* p = static_cast<char*>(base) + off * T::bytes;
  constexpr int PER16 = 16 / T::bytes;   // elements per 16-byte store
  if (nvalid >= N && N % PER16 == 0 && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
    for (int q = 0; q < N; q += PER16) {
      if constexpr (T::bytes == 4) {
        *reinterpret_cast<float4*>(p + 4 * q) =
            make_float4(u[q] * alpha, u[q + 1] * alpha, u[q + 2] * alpha, u[q + 3] * alpha);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = T::pack2(u[q + 2 * j] * alpha, u[q + 2 * j + 1] * alpha);
        *reinterpret_cast<uint4*>(p + 2 * q) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < nvalid) T::store(base, off + q, u[q] * alpha);
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

// One butterfly stage across lanes: lanes l and l^m hold the same positions of the two
// halves; the lane with the bit clear keeps a+b, the other keeps a-b.
template <int N>
__device__ inline void fwht_xlane(float (&v)[N], int lane, int m) {
  const bool upper = (lane & m) != 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float p = xor_lane(v[i], m);
    v[i] = upper ? (p - v[i]) : (v[i] + p);
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
// Scale of a tensor: the given step (STEP mode), or max(partials)/Qp (ABSMAX mode).
// Every thread of the block returns the same (s, r = 1/s, or r = 0 when s == 0).
__device__ inline void tensor_scale(const float* partials, int nparts, const float* step,
                                    int qp, float* red, float& s, float& r) {
  if (step != nullptr) {
    s = *step;
  } else {
    float a = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) a = fmaxf(a, partials[i]);
    a = block_max(a, red);
    s = a / static_cast<float>(qp);   // correctly rounded fp32 division
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

// Pack 4 codes (already in [-127, 127]) into one little-endian dword.
__device__ inline uint32_t pack4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 0xFFu) | ((static_cast<uint32_t>(b) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(c) & 0xFFu) << 16) | ((static_cast<uint32_t>(d) & 0xFFu) << 24);
}

}  // namespace hq
