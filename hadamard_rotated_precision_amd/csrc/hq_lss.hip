// hq_lss.hip — the sampling and bit-split stages of LSS-MM, the sampled weight gradient of the
// INT4-range HQ layer ("Training Transformers with 4-bit Integers": §4.2 bit splitting and
// leverage score sampling, §A.2 the probability procedure, §A.6 the GPU stages, §B.2 the
// unbiased estimator). The integer product that follows is the GEMM of hq_gemm.hip with its
// contraction length read from the device.
//
// Passes, all on one stream:
//   rowmax  max|dY_i| per token and per-workgroup partial maxima (for the INT8 step of dY);
//   score   l_i = ||Q8(dY_i)|| ||qX_i||, one wave per token;
//   prob    one workgroup: the clamp-and-rescale probabilities, the Bernoulli decisions, the
//           ordered list of kept tokens, K' and the bit-split steps;
//   pack    the kept tokens' rows gathered, weighted, split into 14 hi + lo codes and written
//           K-contiguous (D x K'), beside the gathered X codes (C x K'), through LDS tiles;
//           the slots from K' up to the next multiple of 16 are written as zeros.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "hq_device.hpp"
#include "hq_internal.hpp"

namespace hq {
namespace {

constexpr int kWaves = 4;                 // rowmax / score: one wave per token, 4 per block
constexpr int kProbThreads = 1024;        // the single probability workgroup
constexpr int kTileJ = 128;               // pack: kept slots per tile
constexpr int kTileC = 64;                // pack: columns per tile
constexpr int kTilePitch = kTileJ + 16;   // LDS row pitch (bytes) of the transposed tile

int64_t pitch16_of(int64_t n) { return (n + 15) / 16 * 16; }

template <class In>
__device__ inline void load_chunk(const void* row, int64_t d, int64_t n, bool vec, float (&v)[16]) {
  load16<In>(row, d, n, vec && d + 16 <= n, v);
}

// ---------------------------------------------------------------- rowmax
template <class In>
__global__ __launch_bounds__(64 * kWaves) void lss_rowmax_kernel(const void* dy, int64_t N,
                                                                  int64_t D, bool vec,
                                                                  float* rowmax, float* partials) {
  __shared__ float red[32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float bmax = 0.0f;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kWaves + wid; i < N;
       i += static_cast<int64_t>(gridDim.x) * kWaves) {
    const void* row = static_cast<const char*>(dy) + i * D * In::bytes;
    float m = 0.0f;
    for (int64_t d = 16 * lane; d < D; d += 16 * 64) {
      float v[16];
      load_chunk<In>(row, d, D, vec, v);
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    }
    m = wave_max(m);
    if (lane == 0) rowmax[i] = m;
    bmax = fmaxf(bmax, m);
  }
  bmax = block_max(bmax, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = bmax;
}

// ---------------------------------------------------------------- scores
// code = clamp(RNE(v / s), -qp, qp) decided as the exact quotient would be: the fp32 product
// v * fp32(1/s) is within 2^-22 relative of v / s, so away from the midpoints it rounds the
// same way; within 1e-4 of one the quotient is taken in fp64, where an exact midpoint stays
// exact (v and s are fp32) and no other quotient of two fp32 values rounds onto one.
__device__ inline int q_code_f32(float v, float s, float r, int qp) {
  float t = v * r;
  const float a = fabsf(t);
  if (fabsf(a - floorf(a) - 0.5f) < 1e-4f) t = static_cast<float>(rint(static_cast<double>(v) / static_cast<double>(s)));
  const float q = rintf(t);
  return static_cast<int>(fminf(fmaxf(q, -static_cast<float>(qp)), static_cast<float>(qp)));
}

template <class In>
__global__ __launch_bounds__(64 * kWaves) void lss_score_kernel(
    const void* dy, int64_t N, int64_t D, bool vec, const int8_t* qx, int64_t ldx, int64_t C,
    const float* partials, int nparts, double* scores, hq_lss_stats* stats) {
  __shared__ float red[32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = fmaxf(m, partials[i]);
  m = block_max(m, red);
  const float s8 = m / 127.0f;   // correctly rounded fp32 division
  const float r8 = s8 > 0.0f ? 1.0f / s8 : 0.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) stats->s8 = s8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kWaves + wid; i < N;
       i += static_cast<int64_t>(gridDim.x) * kWaves) {
    const void* row = static_cast<const char*>(dy) + i * D * In::bytes;
    int sq = 0;                   // <= 16129 * D / 64 per lane
    for (int64_t d = 16 * lane; d < D; d += 16 * 64) {
      float v[16];
      load_chunk<In>(row, d, D, vec, v);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = s8 > 0.0f ? q_code_f32(v[e], s8, r8, 127) : 0;
        sq += q * q;
      }
    }
    int sx = 0;
    const int8_t* xr = qx + i * ldx;
    for (int64_t c = 16 * lane; c < C; c += 16 * 64) {
      const int4 w = *reinterpret_cast<const int4*>(xr + c);   // ldx % 16 == 0, ldx >= C
      const int words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = static_cast<int8_t>(words[e >> 2] >> (8 * (e & 3)));
        sx += (c + e < C) ? q * q : 0;
      }
    }
    double a = static_cast<double>(sq), b = static_cast<double>(sx);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      a += __shfl_xor(a, o, 64);
      b += __shfl_xor(b, o, 64);
    }
    if (lane == 0) scores[i] = sqrt(a) * sqrt(b);
  }
}

// ---------------------------------------------------------------- probabilities
template <class T>
__device__ inline T prob_block_sum(T x, T* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  T r = red[0];
  for (int w = 1; w < kProbThreads / 64; ++w) r += red[w];
  return r;
}

__device__ inline double prob_block_max(double x, double* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < kProbThreads / 64; ++w) r = fmax(r, red[w]);
  return r;
}

// fp32(m / d) rounded to nearest even from the exact quotient (m >= 0, 1 <= d < 2^20): the
// double quotient rounded to fp32 can be one step off when the double rounding lands on a
// midpoint, so the result is checked against d times the midpoints on either side, which are
// exact in double.
__device__ inline float div_to_f32_exact(double m, double d) {
  float f = static_cast<float>(m / d);
  if (!(f > 0.0f)) return f;
  const uint32_t b = __float_as_uint(f);
  const float up = __uint_as_float(b + 1), dn = __uint_as_float(b - 1);
  const double hi = 0.5 * (static_cast<double>(f) + static_cast<double>(up)) * d;
  const double lo = 0.5 * (static_cast<double>(f) + static_cast<double>(dn)) * d;
  if (m > hi || (m == hi && (b & 1u))) return up;
  if (m < lo || (m == lo && (b & 1u))) return dn;
  return f;
}

// One workgroup. fixed / probs / scores are indexed i = threadIdx.x + 1024 t, so each entry is
// read and written by one thread only; the block sums are the only exchange.
__global__ __launch_bounds__(kProbThreads) void lss_prob_kernel(
    const double* scores, int64_t N, double budget, const float* uniforms, const float* rowmax,
    double* probs, uint8_t* fixed, int32_t* kept_idx, hq_lss_stats* stats) {
  __shared__ double redd[kProbThreads / 64];
  __shared__ int redi[kProbThreads / 64];
  __shared__ int wave_cnt[kProbThreads / 64];
  const int tid = threadIdx.x;
  for (int64_t i = tid; i < N; i += kProbThreads) {
    probs[i] = 0.0;
    fixed[i] = 0;
  }
  for (;;) {
    double tot = 0.0;
    int nfree = 0, nfix = 0;
    for (int64_t i = tid; i < N; i += kProbThreads) {
      if (fixed[i]) {
        ++nfix;
      } else if (scores[i] > 0.0) {
        tot += scores[i];
        ++nfree;
      }
    }
    tot = prob_block_sum(tot, redd);
    nfree = prob_block_sum(nfree, redi);
    nfix = prob_block_sum(nfix, redi);
    const double left = budget - static_cast<double>(nfix);
    if (nfree == 0 || !(left > 0.0)) break;
    int over = 0;
    for (int64_t i = tid; i < N; i += kProbThreads) {
      if (fixed[i] || !(scores[i] > 0.0)) continue;
      double v = left * scores[i] / tot;
      if (v > 1.0) {
        v = 1.0;
        fixed[i] = 1;
        ++over;
      }
      probs[i] = v;
    }
    if (prob_block_sum(over, redi) == 0) break;
  }
  // Bernoulli decisions and the ordered list of kept tokens, 1024 tokens at a time
  const int lane = tid & 63, wid = tid >> 6;
  int base = 0;
  double gmax = 0.0;   // max over kept tokens of max|dY_i| / p_i
  for (int64_t c0 = 0; c0 < N; c0 += kProbThreads) {
    const int64_t i = c0 + tid;
    bool keep = false;
    if (i < N) {
      const double p = probs[i];
      keep = static_cast<double>(uniforms[i]) < p;
      if (keep) gmax = fmax(gmax, static_cast<double>(rowmax[i]) / p);
    }
    const uint64_t bal = __ballot(keep);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wave_cnt[wid] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kProbThreads / 64; ++w) {
      before += (w < wid) ? wave_cnt[w] : 0;
      total += wave_cnt[w];
    }
    if (keep) kept_idx[base + before + rank] = static_cast<int32_t>(i);
    base += total;
  }
  gmax = prob_block_max(gmax, redd);
  if (tid == 0) {
    const float s_hi = div_to_f32_exact(gmax, 7.0);
    stats->kept = base;
    stats->s_hi = s_hi;
    stats->s_lo = static_cast<float>(static_cast<double>(s_hi) / 14.0);
  }
}

// ---------------------------------------------------------------- bit split + gather
// code = clamp(RNE(v / s), -7, 7) decided as the exact quotient would be, up to quotients
// within one fp64 step of a midpoint: the product with the fp64 reciprocal is taken away from
// midpoints, the correctly rounded fp64 quotient near them (exact midpoints stay exact).
__device__ inline double q7_f64(double v, double s, double r) {
  double t = v * r;
  const double a = fabs(t);
  if (fabs(a - floor(a) - 0.5) < 1e-9) t = v / s;
  return fmin(fmax(rint(t), -7.0), 7.0);
}

// blockIdx.y < ty_d: tiles of the split codes of dY (D rows); the rest: tiles of the gathered
// X codes (C rows). Each tile covers kTileJ kept slots x kTileC rows of the output.
template <class In>
__global__ __launch_bounds__(256) void lss_pack_kernel(
    const void* dy, int64_t N, int64_t D, bool vec, const int8_t* qx, int64_t ldx, int64_t C,
    const double* probs, const int32_t* kept_idx, const hq_lss_stats* stats, int ty_d,
    int8_t* ct, int8_t* xt, int64_t ldk) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileC * kTilePitch];
  const int kept = stats->kept;
  const int kpad = (kept + 15) & ~15;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kTileJ;
  if (j0 >= kpad) return;
  const int t = threadIdx.x;
  const bool split = static_cast<int>(blockIdx.y) < ty_d;
  const int64_t c0 = static_cast<int64_t>(split ? blockIdx.y : blockIdx.y - ty_d) * kTileC;
  const int64_t rows_out = split ? D : C;
  if (split) {
    const float s_hi = stats->s_hi, s_lo = stats->s_lo;
    const double shi = s_hi, slo = s_lo;
    const double rhi = s_hi > 0.0f ? 1.0 / shi : 0.0, rlo = s_lo > 0.0f ? 1.0 / slo : 0.0;
    // 8 threads per slot, 8 columns each; 32 slots per pass
    const int rr = t >> 3, cc = (t & 7) * 8;
    for (int pass = 0; pass < kTileJ / 32; ++pass) {
      const int jl = pass * 32 + rr;
      const int64_t j = j0 + jl;
      int code[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (j < kept) {
        const int64_t i = kept_idx[j];
        const double p = probs[i];
        const char* row = static_cast<const char*>(dy) + i * D * In::bytes;
        float v[8];
        const int64_t d = c0 + cc;
        if (vec && d + 8 <= D) {
          if constexpr (In::bytes == 4) {
            const float4 a = *reinterpret_cast<const float4*>(row + d * 4);
            const float4 b = *reinterpret_cast<const float4*>(row + d * 4 + 16);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
          } else {
            const uint4 u = *reinterpret_cast<const uint4*>(row + d * 2);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[2 * e] = In::from_bits(static_cast<uint16_t>(w[e] & 0xFFFFu));
              v[2 * e + 1] = In::from_bits(static_cast<uint16_t>(w[e] >> 16));
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (d + e < D) ? In::load(row, d + e) : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double gw = static_cast<double>(v[e]) / p;
          const double hi = q7_f64(gw, shi, rhi);
          const double lo = q7_f64(gw - shi * hi, slo, rlo);
          code[e] = 14 * static_cast<int>(hi) + static_cast<int>(lo);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[(cc + e) * kTilePitch + jl] = static_cast<uint8_t>(code[e]);
    }
  } else {
    // 4 threads per slot, 16 code bytes each; 64 slots per pass
    const int rr = t >> 2, cc = (t & 3) * 16;
    for (int pass = 0; pass < kTileJ / 64; ++pass) {
      const int jl = pass * 64 + rr;
      const int64_t j = j0 + jl;
      int4 w = make_int4(0, 0, 0, 0);
      if (j < kept && c0 + cc < C) {
        const int64_t i = kept_idx[j];
        w = *reinterpret_cast<const int4*>(qx + i * ldx + c0 + cc);   // within the pitch
      }
      const uint32_t words[4] = {static_cast<uint32_t>(w.x), static_cast<uint32_t>(w.y),
                                 static_cast<uint32_t>(w.z), static_cast<uint32_t>(w.w)};
#pragma unroll
      for (int e = 0; e < 16; ++e)
        tile[(cc + e) * kTilePitch + jl] = static_cast<uint8_t>(words[e >> 2] >> (8 * (e & 3)));
    }
  }
  __syncthreads();
  // write out: 8 threads per output row, 16 slot bytes each; 32 rows per pass
  int8_t* dst = split ? ct : xt;
  const int rr = t >> 3, jc = (t & 7) * 16;
  for (int pass = 0; pass < kTileC / 32; ++pass) {
    const int rl = pass * 32 + rr;
    const int64_t row = c0 + rl;
    if (row < rows_out && j0 + jc < kpad)
      *reinterpret_cast<uint4*>(dst + row * ldk + j0 + jc) =
          *reinterpret_cast<const uint4*>(tile + rl * kTilePitch + jc);
  }
}

template <class In>
hipError_t lss_launch(const LssPass& p, hipStream_t st) {
  const int eb = In::bytes;
  const bool vec = (reinterpret_cast<uintptr_t>(p.dy) & 15u) == 0 && (p.D * eb) % 16 == 0;
  const int64_t row_blocks = (p.N + kWaves - 1) / kWaves;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(row_blocks, kMaxPartials)));
  const double dy_bytes = static_cast<double>(p.N) * p.D * eb;
  int tok = prof_open(K_MISC, dy_bytes);
  hipError_t e = launch_k(lss_rowmax_kernel<In>, dim3(grid), dim3(64 * kWaves), st, tok, p.dy,
                          p.N, p.D, vec, p.rowmax, p.partials);
  if (e != hipSuccess) return e;
  tok = prof_open(K_MISC, dy_bytes + static_cast<double>(p.N) * p.C);
  e = launch_k(lss_score_kernel<In>, dim3(grid), dim3(64 * kWaves), st, tok, p.dy, p.N, p.D, vec,
               p.qx, p.ldx, p.C, static_cast<const float*>(p.partials), grid, p.scores, p.stats);
  if (e != hipSuccess) return e;
  tok = prof_open(K_MISC, static_cast<double>(p.N) * 8.0);
  e = launch_k(lss_prob_kernel, dim3(1), dim3(kProbThreads), st, tok,
               static_cast<const double*>(p.scores), p.N, p.budget, p.uniforms,
               static_cast<const float*>(p.rowmax), p.probs, p.fixed, p.kept_idx, p.stats);
  if (e != hipSuccess) return e;
  const int ty_d = static_cast<int>((p.D + kTileC - 1) / kTileC);
  const int ty_c = static_cast<int>((p.C + kTileC - 1) / kTileC);
  const int64_t tx = (pitch16_of(p.N) + kTileJ - 1) / kTileJ;
  if (tx == 0 || ty_d + ty_c == 0) return hipSuccess;
  tok = prof_open(K_MISC, static_cast<double>(p.N) * (p.D * eb + p.C + p.D + p.C));
  return launch_k(lss_pack_kernel<In>, dim3(static_cast<unsigned>(tx), ty_d + ty_c), dim3(256), st,
                  tok, p.dy, p.N, p.D, vec, p.qx, p.ldx, p.C, static_cast<const double*>(p.probs),
                  static_cast<const int32_t*>(p.kept_idx), static_cast<const hq_lss_stats*>(p.stats),
                  ty_d, p.ct, p.xt, p.ldk);
}

}  // namespace

hipError_t lss_pass(const LssPass& p, hipStream_t st) {
  switch (p.dt) {
    case DT_F32: return lss_launch<F32>(p, st);
    case DT_F16: return lss_launch<F16>(p, st);
    case DT_BF16: return lss_launch<BF16>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hq
