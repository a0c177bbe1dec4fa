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
#include "hq_launch.hpp"

namespace hq {
namespace {

constexpr int kWaves = 4;                 // rowmax / score: one wave per token, 4 per block
constexpr int kProbThreads = 256;         // the probability workgroup with tokens in registers
constexpr int kProbThreadsMem = 1024;     // ... with tokens in memory (N > 32 kProbThreads)
constexpr int kTileJ = 128;               // pack: kept slots per tile
constexpr int kTileC = 64;                // pack: columns per tile
constexpr int kTilePitch = kTileJ + 16;   // LDS row pitch (bytes) of the transposed tile

int64_t pitch16_of(int64_t n) { return (n + 15) / 16 * 16; }

// Calls f(v) for each 16-element chunk of a row of D elements that lane `lane` of a wave owns
// (chunks at 16 lane + 1024 s). Whole strides of the wave go in groups of four, with all four
// loads issued before any is used; the last partial stride is read with bounds checks (as is
// everything when vec is false: the row is not 16-byte aligned).
template <class In, class F>
__device__ inline void row_chunks(const void* row, int64_t D, bool vec, int lane, F&& f) {
  const int64_t full = vec ? D / 1024 : 0;
  int64_t s = 0;
  for (; s + 4 <= full; s += 4) {
    float v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) load16<In>(row, (s + u) * 1024 + 16 * lane, D, true, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) f(v[u]);
  }
  for (; s < full; ++s) {
    float v[16];
    load16<In>(row, s * 1024 + 16 * lane, D, true, v);
    f(v);
  }
  for (int64_t d = s * 1024 + 16 * lane; d < D; d += 1024) {
    float v[16];
    load16<In>(row, d, D, vec && d + 16 <= D, v);
    f(v);
  }
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
    row_chunks<In>(row, D, vec, lane, [&](const float (&v)[16]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    });
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
    // the X codes of the token (one 16-byte chunk per lane for C <= 1024) go out first, so
    // their load overlaps the dY loads
    const int8_t* xr = qx + i * ldx;
    int4 x0 = make_int4(0, 0, 0, 0);
    if (16 * lane < C) x0 = *reinterpret_cast<const int4*>(xr + 16 * lane);   // ldx % 16 == 0, ldx >= C
    int sq = 0;                   // <= 16129 * D / 64 per lane
    row_chunks<In>(row, D, vec, lane, [&](const float (&v)[16]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = s8 > 0.0f ? q_code_f32(v[e], s8, r8, 127) : 0;
        sq += q * q;
      }
    });
    int sx = 0;
    for (int64_t c = 16 * lane; c < C; c += 16 * 64) {
      const int4 w = c == 16 * lane ? x0 : *reinterpret_cast<const int4*>(xr + c);
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
template <int NT>
__device__ inline double prob_block_max(double x, double* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < NT / 64; ++w) r = fmax(r, red[w]);
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

// Workgroup sums of one round, in a fixed order (lane tree, then the waves in order); every
// thread gets the totals. The two counts travel packed in one 64-bit word (each < 2^32).
template <int NT>
__device__ inline void prob_round_sums(double& tot, int& nfree, int& nfix, double* red,
                                       uint64_t* redc) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint64_t cnt = static_cast<uint64_t>(static_cast<uint32_t>(nfree)) |
                 (static_cast<uint64_t>(static_cast<uint32_t>(nfix)) << 32);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    tot += __shfl_xor(tot, o, 64);
    cnt += __shfl_xor(cnt, o, 64);
  }
  if (lane == 0) {
    red[wid] = tot;
    redc[wid] = cnt;
  }
  __syncthreads();
  tot = red[0];
  cnt = redc[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    tot += red[w];
    cnt += redc[w];
  }
  nfree = static_cast<int>(cnt & 0xFFFFFFFFu);
  nfix = static_cast<int>(cnt >> 32);
  __syncthreads();   // every thread has read red / redc before the next round writes them
}

// One workgroup of NT threads; token i = threadIdx.x + NT t belongs to one thread, which alone
// reads and writes its score, clamp flag and probability. PT > 0: the scores are held in
// registers and the clamp flags in a bit mask (N <= NT PT); PT = 0: the `scores`, `fixed` and
// `probs` arrays, read a batch of 8 at a time.
//
// Each round sums the free scores and counts the free and clamped tokens, then assigns
// p = (left / sum) l to the free tokens, clamping those above 1. A round whose sums show no
// token clamped since the previous round ends the loop with the previous assignment standing
// (that assignment clamped nothing): the same sequence of assignments as testing for clamps
// right after each one, with one workgroup reduction per round. With the scores in registers
// the final p follow from the last round's scale: 1 if clamped, scale l if free, 0 otherwise.
template <int NT, int PT>
__global__ __launch_bounds__(NT) void lss_prob_kernel(
    const double* scores, int64_t N, double budget, const float* uniforms, const float* rowmax,
    double* probs, uint8_t* fixed, int32_t* kept_idx, double* kept_p, hq_lss_stats* stats) {
  constexpr bool REG = PT > 0;
  constexpr int R = REG ? PT : 1;
  constexpr int NW = NT / 64;
  constexpr int B = 8;   // PT = 0: tokens per batch of loads
  __shared__ double redd[NW];
  __shared__ uint64_t redc[NW];
  __shared__ int wave_cnt[(REG ? PT : 1) * NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  if (N <= 0) {
    if (tid == 0) {
      stats->kept = 0;
      stats->s_hi = 0.0f;
      stats->s_lo = 0.0f;
    }
    return;
  }
  double sc[R];
  uint32_t fxm = 0;   // REG: bit t = token t clamped
  if constexpr (REG) {
    // loads at clamped indices (N >= 1 here), all issued before any is used; the entries past
    // N are then masked
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int64_t i = tid + static_cast<int64_t>(NT) * t;
      sc[t] = scores[i < N ? i : N - 1];
    }
#pragma unroll
    for (int t = 0; t < PT; ++t)
      if (tid + static_cast<int64_t>(NT) * t >= N) sc[t] = 0.0;
  } else {
    for (int64_t i = tid; i < N; i += NT) {
      probs[i] = 0.0;
      fixed[i] = 0;
    }
  }
  int prev_fix = -1;
  double c_last = 0.0;   // REG: the scale of the last assignment (0: none yet)
  for (;;) {
    double tot = 0.0;
    int nfree = 0, nfix = 0;
    if constexpr (REG) {
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        if ((fxm >> t) & 1u) {
          ++nfix;
        } else if (sc[t] > 0.0) {
          tot += sc[t];
          ++nfree;
        }
      }
    } else {
      for (int64_t i0 = tid; i0 < N; i0 += static_cast<int64_t>(NT) * B) {
        double v[B];
        uint8_t f[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int64_t i = i0 + static_cast<int64_t>(NT) * b;
          v[b] = scores[i < N ? i : N - 1];
          f[b] = fixed[i < N ? i : N - 1];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          if (i0 + static_cast<int64_t>(NT) * b >= N) continue;
          if (f[b]) {
            ++nfix;
          } else if (v[b] > 0.0) {
            tot += v[b];
            ++nfree;
          }
        }
      }
    }
    prob_round_sums<NT>(tot, nfree, nfix, redd, redc);
    const double left = budget - static_cast<double>(nfix);
    if (nfree == 0 || !(left > 0.0) || nfix == prev_fix) break;
    prev_fix = nfix;
    const double c = left / tot;   // the round's scale: p = c l
    if constexpr (REG) {
      c_last = c;
#pragma unroll
      for (int t = 0; t < PT; ++t)
        if (!((fxm >> t) & 1u) && c * sc[t] > 1.0) fxm |= 1u << t;
    } else {
      for (int64_t i0 = tid; i0 < N; i0 += static_cast<int64_t>(NT) * B) {
        double v[B];
        uint8_t f[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int64_t i = i0 + static_cast<int64_t>(NT) * b;
          v[b] = scores[i < N ? i : N - 1];
          f[b] = fixed[i < N ? i : N - 1];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int64_t i = i0 + static_cast<int64_t>(NT) * b;
          if (i >= N || f[b] || !(v[b] > 0.0)) continue;
          double q = c * v[b];
          if (q > 1.0) {
            q = 1.0;
            fixed[i] = 1;
          }
          probs[i] = q;
        }
      }
    }
  }
  // Bernoulli decisions and the ordered list of kept tokens
  int base = 0;
  double gmax = 0.0;   // max over kept tokens of max|dY_i| / p_i
  if constexpr (REG) {
    float uf[PT], rm[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int64_t i = tid + static_cast<int64_t>(NT) * t;
      uf[t] = uniforms[i < N ? i : N - 1];
      rm[t] = rowmax[i < N ? i : N - 1];
    }
    // every chunk's ballot first, then one barrier, then each thread places its kept tokens
    uint64_t bal[PT];
    double pr[PT];
    uint32_t keepm = 0;
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int64_t i = tid + static_cast<int64_t>(NT) * t;
      pr[t] = ((fxm >> t) & 1u) ? 1.0 : (sc[t] > 0.0 ? c_last * sc[t] : 0.0);
      const bool keep = i < N && static_cast<double>(uf[t]) < pr[t];
      if (keep) {
        keepm |= 1u << t;
        gmax = fmax(gmax, static_cast<double>(rm[t]) / pr[t]);
      }
      if (i < N) probs[i] = pr[t];
      bal[t] = __ballot(keep);
      if (lane == 0) wave_cnt[t * NW + wid] = __popcll(bal[t]);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cw = wave_cnt[t * NW + w];
        before += (w < wid) ? cw : 0;
        total += cw;
      }
      if ((keepm >> t) & 1u) {
        const int pos = base + before + __popcll(bal[t] & ((1ull << lane) - 1ull));
        kept_idx[pos] = static_cast<int32_t>(tid + NT * t);
        kept_p[pos] = pr[t];
      }
      base += total;
    }
  } else {
    const int64_t T = (N + NT - 1) / NT;
    for (int64_t t = 0; t < T; ++t) {
      const int64_t i = tid + static_cast<int64_t>(NT) * t;
      bool keep = false;
      double p = 0.0;
      if (i < N) {
        p = probs[i];
        keep = static_cast<double>(uniforms[i]) < p;
        if (keep) gmax = fmax(gmax, static_cast<double>(rowmax[i]) / p);
      }
      const uint64_t bal = __ballot(keep);
      if (lane == 0) wave_cnt[wid] = __popcll(bal);
      __syncthreads();
      int before = 0, total = 0;
      for (int w = 0; w < NW; ++w) {
        before += (w < wid) ? wave_cnt[w] : 0;
        total += wave_cnt[w];
      }
      if (keep) {
        const int pos = base + before + __popcll(bal & ((1ull << lane) - 1ull));
        kept_idx[pos] = static_cast<int32_t>(i);
        kept_p[pos] = p;
      }
      base += total;
      __syncthreads();   // the counts are read before the next chunk writes them
    }
  }
  gmax = prob_block_max<NT>(gmax, redd);
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

// Eight consecutive elements of a row from element d on (zeros past n); vec: the row base is
// 16-byte aligned and the row length a multiple of 16 bytes.
template <class In>
__device__ inline void load8(const char* row, int64_t d, int64_t n, bool vec, float (&v)[8]) {
  if (vec && d + 8 <= n) {
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
    for (int e = 0; e < 8; ++e) v[e] = (d + e < n) ? In::load(row, d + e) : 0.0f;
  }
}

// The combined code 14 hi + lo of one element g of a kept row with probability p:
// gw = fp64(g / p), hi = Q7(gw / s_hi), lo = Q7((gw - s_hi hi) / s_lo), each rounding decided
// as the exact quotient would be. Fast path in fp32: gw ~ g * fp32(1/p) is within 1.3e-7
// relative of gw, so t_hi = gw / s_hi comes out within 3e-6 and t_lo = (gw - s_hi hi) / s_lo
// (s_hi / s_lo ~ 14) within 1.5e-5 of their exact values; a decision that such an error cannot
// flip (both quotients more than 1e-4 from a midpoint) is the exact one. Otherwise the fp64
// path decides.
struct SplitSteps {
  float s_hi, s_lo, r_hi, r_lo;   // fp32 steps and reciprocals
  double shi, slo, rhi, rlo;      // the same in fp64
};

__device__ inline int split_code(float g, double p, float w, const SplitSteps& k) {
  const float gw = g * w;
  const float th = gw * k.r_hi;
  const float hi = rintf(th);
  const float tl = __builtin_fmaf(-k.s_hi, hi, gw) * k.r_lo;
  const float lo = rintf(tl);
  const float ah = fabsf(th), al = fabsf(tl);
  if (fabsf(ah - floorf(ah) - 0.5f) >= 1e-4f && fabsf(al - floorf(al) - 0.5f) >= 1e-4f)
    return 14 * static_cast<int>(fminf(fmaxf(hi, -7.0f), 7.0f)) +
           static_cast<int>(fminf(fmaxf(lo, -7.0f), 7.0f));
  const double gd = static_cast<double>(g) / p;
  const double h = q7_f64(gd, k.shi, k.rhi);
  const double l = q7_f64(gd - k.shi * h, k.slo, k.rlo);
  return 14 * static_cast<int>(h) + static_cast<int>(l);
}

// blockIdx.y < ty_d: tiles of the split codes of dY (D rows); the rest: tiles of the gathered
// X codes (C rows). Each tile covers kTileJ kept slots x kTileC rows of the output. Every
// thread first loads the kept-token indices (and probabilities) of all its slots, then all
// its row chunks, so the gathers of one thread are in flight together.
template <class In>
__global__ __launch_bounds__(256) void lss_pack_kernel(
    const void* dy, int64_t N, int64_t D, bool vec, const int8_t* qx, int64_t ldx, int64_t C,
    const int32_t* kept_idx, const double* kept_p, const hq_lss_stats* stats, int ty_d,
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
    constexpr int NP = kTileJ / 32;   // 8 threads per slot, 8 columns each, 32 slots per pass
    SplitSteps ks;
    ks.s_hi = stats->s_hi;
    ks.s_lo = stats->s_lo;
    ks.r_hi = ks.s_hi > 0.0f ? 1.0f / ks.s_hi : 0.0f;
    ks.r_lo = ks.s_lo > 0.0f ? 1.0f / ks.s_lo : 0.0f;
    ks.shi = ks.s_hi;
    ks.slo = ks.s_lo;
    ks.rhi = ks.s_hi > 0.0f ? 1.0 / ks.shi : 0.0;
    ks.rlo = ks.s_lo > 0.0f ? 1.0 / ks.slo : 0.0;
    const int rr = t >> 3, cc = (t & 7) * 8;
    const int64_t d = c0 + cc;
    // every load at a clamped (valid) slot and column, all issued before any is used; slots
    // past K' and columns past D are masked afterwards (kept >= 1 here)
    int64_t tok[NP];
    double p[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int64_t j = min(j0 + q * 32 + rr, static_cast<int64_t>(kept) - 1);
      tok[q] = kept_idx[j];
      p[q] = kept_p[j];
    }
    float v[NP][8];
#pragma unroll
    for (int q = 0; q < NP; ++q)
      load8<In>(static_cast<const char*>(dy) + tok[q] * D * In::bytes, d, D, vec, v[q]);
#pragma unroll
    for (int q = 0; q < NP; ++q)
      if (j0 + q * 32 + rr >= kept)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = 0.0f;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int jl = q * 32 + rr;
      const float w = static_cast<float>(1.0 / p[q]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tile[(cc + e) * kTilePitch + jl] = static_cast<uint8_t>(split_code(v[q][e], p[q], w, ks));
    }
  } else {
    constexpr int NP = kTileJ / 64;   // 4 threads per slot, 16 code bytes each, 64 slots per pass
    const int rr = t >> 2, cc = (t & 3) * 16;
    int4 w[NP];
    int64_t tok[NP];
    // clamped slot and column chunk (c0 < C, so chunk c0 is valid), loads first, masks after;
    // a chunk starting below C ends within the pitch (C <= ldx, both multiples of 16)
    const int64_t col = c0 + cc < C ? c0 + cc : c0;
#pragma unroll
    for (int q = 0; q < NP; ++q)
      tok[q] = kept_idx[min(j0 + q * 64 + rr, static_cast<int64_t>(kept) - 1)];
#pragma unroll
    for (int q = 0; q < NP; ++q) w[q] = *reinterpret_cast<const int4*>(qx + tok[q] * ldx + col);
#pragma unroll
    for (int q = 0; q < NP; ++q)
      if (j0 + q * 64 + rr >= kept || c0 + cc >= C) w[q] = make_int4(0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int jl = q * 64 + rr;
      const uint32_t words[4] = {static_cast<uint32_t>(w[q].x), static_cast<uint32_t>(w[q].y),
                                 static_cast<uint32_t>(w[q].z), static_cast<uint32_t>(w[q].w)};
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

hipError_t prob_launch(const LssPass& p, hipStream_t st, int tok) {
  auto go = [&](auto kernel, int nt) {
    return launch_k(kernel, dim3(1), dim3(nt), st, tok, static_cast<const double*>(p.scores), p.N,
                    p.budget, p.uniforms, static_cast<const float*>(p.rowmax), p.probs, p.fixed,
                    p.kept_idx, p.kept_p, p.stats);
  };
  constexpr int T = kProbThreads;
  if (p.N <= 4 * T) return go(lss_prob_kernel<T, 4>, T);
  if (p.N <= 8 * T) return go(lss_prob_kernel<T, 8>, T);
  if (p.N <= 16 * T) return go(lss_prob_kernel<T, 16>, T);
  if (p.N <= 32 * T) return go(lss_prob_kernel<T, 32>, T);
  return go(lss_prob_kernel<kProbThreadsMem, 0>, kProbThreadsMem);
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
  e = prob_launch(p, st, prof_open(K_MISC, static_cast<double>(p.N) * 8.0));
  if (e != hipSuccess) return e;
  const int ty_d = static_cast<int>((p.D + kTileC - 1) / kTileC);
  const int ty_c = static_cast<int>((p.C + kTileC - 1) / kTileC);
  const int64_t tx = (pitch16_of(p.N) + kTileJ - 1) / kTileJ;
  if (tx == 0 || ty_d + ty_c == 0) return hipSuccess;
  tok = prof_open(K_MISC, static_cast<double>(p.N) * (p.D * eb + p.C + p.D + p.C));
  return launch_k(lss_pack_kernel<In>, dim3(static_cast<unsigned>(tx), ty_d + ty_c), dim3(256), st,
                  tok, p.dy, p.N, p.D, vec, p.qx, p.ldx, p.C,
                  static_cast<const int32_t*>(p.kept_idx), static_cast<const double*>(p.kept_p),
                  static_cast<const hq_lss_stats*>(p.stats), ty_d, p.ct, p.xt, p.ldk);
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
