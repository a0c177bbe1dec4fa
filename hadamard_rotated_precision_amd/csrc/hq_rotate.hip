// hq_rotate.hip — the standalone block-diagonal Walsh-Hadamard transform (floating point in,
// floating point out) behind hq_fwht, and the small fill kernels of the library.
//
// "Training Transformers with 4-bit Integers", §3.3 (the block-diagonal H_k transform that
// spreads outliers before quantization); "HALO: Hadamard-Assisted Lower-Precision Optimization
// for LLMs", Approach (right rotation along the hidden axis, left rotation along the token
// axis). The quantizing prologues of the layer calls live in hq_prologue.hip; these kernels
// write the rotated values themselves.
//
// Two transform shapes, both streaming with 16-byte loads and stores:
//   rows kernel  — rotation along the contiguous axis (RIGHT). A 16-lane group owns a 256-column
//                  segment of one row; each lane owns 16 consecutive elements, so strides < 16
//                  are in-register butterflies and strides 16..128 are lane exchanges.
//   cols kernel  — rotation along the row axis (LEFT, the token axis). A workgroup stages a
//                  KL-row tile in LDS (fp32, column-swizzled), each thread owns KL/P consecutive
//                  rows of one column (in-register stages) and P lanes share a column; the tile
//                  goes back through LDS so the stores are row-contiguous.
#include <algorithm>

#include <cstdlib>

#include "hq_device.hpp"
#include "hq_internal.hpp"
#include "hq_launch.hpp"

namespace hq {

constexpr int kThreads = 256;

// ============================================================ rows kernel (RIGHT / NONE)
struct RowArgs {
  const void* src;
  int64_t rows, cols;   // src is rows x cols, row pitch = cols elements
  bool vec;             // 16-byte loads are legal for every full 16-element chunk
  void* dst;            // rows x cols output (pitch cols)
  int nt;               // output stores carry the non-temporal hint
};

template <class In, class Out, int KR>
__global__ __launch_bounds__(kThreads) void rows_kernel(RowArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = lane & 15;                        // lane within the 16-lane group
  const int group = (blockIdx.x * kThreads + threadIdx.x) >> 4;
  const int ngroups = (gridDim.x * kThreads) >> 4;
  const int64_t nseg = (a.cols + 255) / 256;
  const int64_t items = a.rows * nseg;

  // Every lane runs the same number of iterations so the lane exchanges stay convergent.
  const int64_t iters = (items + ngroups - 1) / ngroups;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t item = group + it * ngroups;
    const bool live = item < items;
    const int64_t row = live ? item / nseg : 0;
    const int64_t c0 = live ? (item % nseg) * 256 + 16 * g : a.cols;   // first column
    const char* rowp = static_cast<const char*>(a.src) + row * a.cols * In::bytes;
    float v[16];
    const bool full = c0 + 16 <= a.cols;
    load16<In>(rowp, c0, live ? a.cols : 0, a.vec && full, v);

    fwht_inreg<KR, 16>(v);
#pragma unroll
    for (int m = 1; 16 * m < KR; m <<= 1) fwht_xlane<16>(v, g, m);

    if (!live || c0 >= a.cols) continue;
    // 16-byte stores when the run is whole and aligned, element stores otherwise
    if (a.nt) store_run<Out, 16, false, true>(a.dst, row * a.cols + c0, a.cols - c0, v, 1.0f);
    else store_run<Out, 16>(a.dst, row * a.cols + c0, a.cols - c0, v, 1.0f);
  }
}

// ============================================================ rotated statistics
// One pass over a right-rotated tensor R = V B (and, for the step gradient, the rotated
// gradient G B) reducing one per-element term ("Training Transformers with 4-bit Integers",
// §A.3 step gradients from cheap elementwise residuals, §A.4 cold-start steps, §A.5 the
// Hadamard size minimising the quantization errors):
//   STAT_ABS_SUM  |v|              STAT_ABS_MAX  max |v| (the absmax of a candidate size)
//   STAT_QERR     (v - s q(v))^2   q: the library's quantizer (integer or E4M3 codes)
//   STAT_LSQ      (g / k) dv_hat/ds, dv_hat/ds = q - v/s inside the grid, +-Qp clipped
// Layout as rows_kernel: a 16-lane group owns a 256-column segment of one row, 16 consecutive
// elements per lane. Each thread sums in fp64; per-workgroup partials (fp64) are reduced in a
// fixed order by stat_finish_kernel, so results do not depend on scheduling.
enum StatMode : int { STAT_ABS_SUM = 0, STAT_QERR = 1, STAT_LSQ = 2, STAT_ABS_MAX = 3 };

struct StatArgs {
  const void* src;
  const void* grad;       // STAT_LSQ: gradient with respect to V (same shape and dtype)
  int64_t rows, cols;
  bool vec;
  const float* scale;     // STAT_QERR / STAT_LSQ: the step s
  int qp;
  float inv_k;            // STAT_LSQ: 1 / k (the gradient with respect to R is (G B) / k)
  double* partials;       // one per workgroup
};

__device__ inline double block_sum_f64(double x, double* red, bool take_max) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double y = __shfl_xor(x, m, 64);
    x = take_max ? fmax(x, y) : x + y;
  }
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < nw; ++w) r = take_max ? fmax(r, red[w]) : r + red[w];
  return r;
}

// VEC: every segment is a whole aligned 256-column run (aligned rows, cols % 256 == 0) and there
// are fewer than 2^31 of them; the segments then stay raw 16-byte chunks while in flight and are
// converted when processed.
template <class In, int KR, int MODE, bool F8, bool VEC>
__global__ __launch_bounds__(kThreads) void stat_kernel(StatArgs a) {
  __shared__ double red[kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int g = lane & 15;
  const int group = (blockIdx.x * kThreads + threadIdx.x) >> 4;
  const int ngroups = (gridDim.x * kThreads) >> 4;
  const int64_t nseg = (a.cols + 255) / 256;
  const int64_t items = a.rows * nseg;
  const int64_t iters = (items + ngroups - 1) / ngroups;
  float s = 0.0f, r = 0.0f;
  double rd = 0.0;
  if constexpr (MODE == STAT_QERR || MODE == STAT_LSQ) {
    s = *a.scale;
    r = (s > 0.0f) ? 1.0f / s : 0.0f;
    rd = (s > 0.0f) ? 1.0 / static_cast<double>(s) : 0.0;
  }
  constexpr bool G = MODE == STAT_LSQ;
  double acc = 0.0;
  // The segments of this group's iterations go through rotating register sets: three in the VEC
  // form, whose raw chunks stay in flight two segments ahead; two in the element form, which
  // converts on load and so waits for its loads there. A segment past the end loads the last
  // one again and is skipped.
  auto fetch = [&](int64_t it, float (&v)[16], float (&gv)[16]) {
    int64_t item = group + it * ngroups;
    if (item >= items) item = items - 1;
    const int64_t row = item / nseg;
    const int64_t c0 = (item % nseg) * 256 + 16 * g;
    const bool full = c0 + 16 <= a.cols;
    load16<In>(static_cast<const char*>(a.src) + row * a.cols * In::bytes, c0, a.cols,
               a.vec && full, v);
    if constexpr (G)
      load16<In>(static_cast<const char*>(a.grad) + row * a.cols * In::bytes, c0, a.cols,
                 a.vec && full, gv);
  };
  auto process = [&](int64_t it, float (&v)[16], float (&gv)[16]) {
    const bool live = group + it * ngroups < items;
    fwht_inreg<KR, 16>(v);
#pragma unroll
    for (int m = 1; 16 * m < KR; m <<= 1) fwht_xlane<16>(v, g, m);
    if constexpr (G) {
      fwht_inreg<KR, 16>(gv);
#pragma unroll
      for (int m = 1; 16 * m < KR; m <<= 1) fwht_xlane<16>(gv, g, m);
    }
    if (!live) return;     // a repeated segment: its terms are not counted
    float part = 0.0f;     // at most 16 terms in fp32, then into the fp64 sum
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (MODE == STAT_ABS_SUM) {
        part += fabsf(v[i]);
      } else if constexpr (MODE == STAT_ABS_MAX) {
        part = fmaxf(part, fabsf(v[i]));
      } else if constexpr (MODE == STAT_QERR) {
        // the difference in fp64 (s times a code is exact there): it cancels most of v
        double level;
        if constexpr (F8) {
          const uint32_t c = e4m3_pack4(v[i], 0.0f, 0.0f, 0.0f, r);
          level = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
        } else {
          level = quant_code(v[i], r, a.qp);
        }
        const double e = static_cast<double>(v[i]) - static_cast<double>(s) * level;
        acc += e * e;
      } else {
        // r / s as a product with the fp64 reciprocal (within 2^-52 of the quotient)
        const double x = static_cast<double>(v[i]) * rd;
        const double d = fabs(x) >= a.qp ? copysign(static_cast<double>(a.qp), x)
                                         : static_cast<double>(quant_code(v[i], r, a.qp)) - x;
        acc += static_cast<double>(gv[i]) * a.inv_k * d;
      }
    }
    if constexpr (MODE == STAT_ABS_SUM) acc += part;
    if constexpr (MODE == STAT_ABS_MAX) acc = fmax(acc, static_cast<double>(part));
  };
  if constexpr (VEC) {
    // 32-bit index arithmetic (the host takes this form only for items < 2^31): a 64-bit
    // division would branch, and the compiler waits for the loads in flight at such branches.
    const uint32_t nseg32 = static_cast<uint32_t>(nseg), last = static_cast<uint32_t>(items - 1);
    auto fetch_raw = [&](int64_t it, uint4 (&q)[4], uint4 (&gq)[4]) {
      const int64_t want = group + it * ngroups;
      const uint32_t item = want < items ? static_cast<uint32_t>(want) : last;
      const uint32_t row = item / nseg32, seg = item - row * nseg32;
      const int64_t off = static_cast<int64_t>(row) * a.cols + 256 * seg + 16 * g;
      load16_raw<In>(a.src, off, q);
      if constexpr (G) load16_raw<In>(a.grad, off, gq);
    };
    auto run = [&](int64_t it, const uint4 (&q)[4], const uint4 (&gq)[4]) {
      float v[16], gv[16];
      unpack16<In>(q, v);
      if constexpr (G) unpack16<In>(gq, gv);
      process(it, v, gv);
    };
    if (items > 0) {   // three register sets: two segments in flight while one is processed
      uint4 qa[4], qb[4], qc[4], ga[4], gb[4], gc[4];
      fetch_raw(0, qa, ga);
      fetch_raw(1, qb, gb);
      for (int64_t it = 0;; it += 3) {
        fetch_raw(it + 2, qc, gc);
        keep_issued();
        run(it, qa, ga);
        if (it + 1 >= iters) break;
        fetch_raw(it + 3, qa, ga);
        keep_issued();
        run(it + 1, qb, gb);
        if (it + 2 >= iters) break;
        fetch_raw(it + 4, qb, gb);
        keep_issued();
        run(it + 2, qc, gc);
        if (it + 3 >= iters) break;
      }
    }
  } else if (items > 0) {
    float va[16], vb[16], ga[G ? 16 : 1], gb[G ? 16 : 1];
    float (&gA)[16] = *reinterpret_cast<float(*)[16]>(G ? ga : va);
    float (&gB)[16] = *reinterpret_cast<float(*)[16]>(G ? gb : vb);
    fetch(0, va, gA);
    int64_t it = 0;
    for (; it + 1 < iters; it += 2) {
      fetch(it + 1, vb, gB);
      process(it, va, gA);
      fetch(it + 2, va, gA);
      process(it + 1, vb, gB);
    }
    if (it < iters) process(it, va, gA);
  }
  acc = block_sum_f64(acc, red, MODE == STAT_ABS_MAX);
  if (threadIdx.x == 0) a.partials[blockIdx.x] = acc;
}

// Reduce the partials in a fixed order into out[0]; then, by `finish`: 0 nothing more; 1 the scale
// max / qp (fp32, for STAT_ABS_MAX: the tensor-wise absmax scale); 2 the cold-start step
// fp32(2 * (sum / n) / sqrt(qp)) into fout.
constexpr int kFinishThreads = 256;

__global__ __launch_bounds__(kFinishThreads) void stat_finish_kernel(
    const double* partials, int nparts, bool take_max, double* out, int finish, double n, int qp,
    float* fout) {
  __shared__ double red[kFinishThreads / 64];
  // thread t takes partials t, t + 256, ... in order; then the lane tree and the waves in order
  double t = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kFinishThreads)
    t = take_max ? fmax(t, partials[i]) : t + partials[i];
  t = block_sum_f64(t, red, take_max);
  if (threadIdx.x != 0) return;
  if (out) *out = t;
  if (finish == 1) *fout = static_cast<float>(t) / static_cast<float>(qp);
  if (finish == 2) *fout = static_cast<float>(2.0 * (t / n) / sqrt(static_cast<double>(qp)));
}

template <class In, int MODE, bool F8>
static hipError_t stat_launch_k(int k, const StatArgs& a, int grid, hipStream_t st, int tok) {
  const bool vec = a.vec && a.cols % 256 == 0 && a.rows * (a.cols / 256) < (int64_t(1) << 31);
  switch (k) {
#define HQ_SK(KK) \
  case KK:                                                                                        \
    return vec ? launch_k(stat_kernel<In, KK, MODE, F8, true>, dim3(grid), dim3(kThreads), st, tok, a) \
               : launch_k(stat_kernel<In, KK, MODE, F8, false>, dim3(grid), dim3(kThreads), st, tok, a);
    HQ_SK(1) HQ_SK(2) HQ_SK(4) HQ_SK(8) HQ_SK(16) HQ_SK(32) HQ_SK(64) HQ_SK(128) HQ_SK(256)
#undef HQ_SK
  }
  return hipErrorInvalidValue;
}

template <class In>
static hipError_t stat_launch_in(int k, int mode, bool f8, const StatArgs& a, int grid,
                                 hipStream_t st, int tok) {
  switch (mode) {
    case STAT_ABS_SUM: return stat_launch_k<In, STAT_ABS_SUM, false>(k, a, grid, st, tok);
    case STAT_ABS_MAX: return stat_launch_k<In, STAT_ABS_MAX, false>(k, a, grid, st, tok);
    case STAT_QERR:
      return f8 ? stat_launch_k<In, STAT_QERR, true>(k, a, grid, st, tok)
                : stat_launch_k<In, STAT_QERR, false>(k, a, grid, st, tok);
    case STAT_LSQ: return stat_launch_k<In, STAT_LSQ, false>(k, a, grid, st, tok);
  }
  return hipErrorInvalidValue;
}

hipError_t stat_pass(const StatPass& p, hipStream_t st) {
  StatArgs a{};
  a.src = p.src;
  a.grad = p.grad;
  a.rows = p.rows;
  a.cols = p.cols;
  const int eb = p.dt == DT_F32 ? 4 : 2;
  a.vec = (reinterpret_cast<uintptr_t>(p.src) & 15u) == 0 && (p.cols * eb) % 16 == 0 &&
          (!p.grad || (reinterpret_cast<uintptr_t>(p.grad) & 15u) == 0);
  a.scale = p.scale;
  a.qp = p.qp;
  a.inv_k = 1.0f / static_cast<float>(p.k);
  a.partials = p.partials;
  const int64_t items = p.rows * ((p.cols + 255) / 256);
  const int64_t groups_per_block = kThreads / 16;
  int64_t grid = (items + groups_per_block - 1) / groups_per_block;
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, kStatMaxParts));
  const double bytes = static_cast<double>(p.rows) * p.cols * eb * (p.grad ? 2 : 1);
  const int tok = prof_open(K_MISC, bytes);
  hipError_t e = hipErrorInvalidValue;
  switch (p.dt) {
    case DT_F32: e = stat_launch_in<F32>(p.k, p.mode, p.f8, a, static_cast<int>(grid), st, tok); break;
    case DT_F16: e = stat_launch_in<F16>(p.k, p.mode, p.f8, a, static_cast<int>(grid), st, tok); break;
    case DT_BF16: e = stat_launch_in<BF16>(p.k, p.mode, p.f8, a, static_cast<int>(grid), st, tok); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stat_finish_kernel, dim3(1), dim3(kFinishThreads), 0, st, p.partials, static_cast<int>(grid),
                     p.mode == STAT_ABS_MAX, p.out, p.finish,
                     static_cast<double>(p.rows) * static_cast<double>(p.cols), p.qp, p.fout);
  return hipGetLastError();
}

// ============================================================ cols kernel (LEFT)
struct ColArgs {
  const void* src;
  int64_t rows, cols;   // rows % KL == 0
  bool vec;             // 16-byte loads are aligned (row pitch a multiple of 16 bytes, base aligned)
  void* dst;            // rows x cols output
  int nt;               // output stores carry the non-temporal hint
};

template <int KL> struct ColShape {
  static constexpr int P = KL >= 4 ? 4 : KL;      // lanes sharing one column
  static constexpr int M = KL / P;                // rows per thread
  static constexpr int NC = kThreads / P;         // columns per tile
};

template <class In, class Out, int KL>
__global__ __launch_bounds__(kThreads) void cols_kernel(ColArgs a) {
  using S = ColShape<KL>;
  constexpr int P = S::P, M = S::M, NC = S::NC;
  constexpr int E = 16 / In::bytes;               // elements per 16-byte load
  __shared__ __attribute__((aligned(16))) float tile[KL * NC];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int c = t / P, p = t % P;
  const int64_t nrb = a.rows / KL;
  const int64_t ncb = (a.cols + NC - 1) / NC;
  const int64_t tiles = nrb * ncb;
  // element (row, col) of the tile lives at row*NC + (col ^ (16 * (row / M))): the column
  // phase's reads (lanes = 16 columns x P row groups) meet 64 distinct banks, and runs of 16
  // columns stay contiguous for the row phases' 16-byte accesses
  auto slot = [](int row, int col) { return row * NC + (col ^ (16 * (row / M))); };

  for (int64_t tile_id = blockIdx.x; tile_id < tiles; tile_id += gridDim.x) {
    const int64_t r0 = (tile_id / ncb) * KL;
    const int64_t col0 = (tile_id % ncb) * NC;
    __syncthreads();
    // stage KL x NC values, one 16-byte load (E consecutive columns) per thread per step
    for (int q = t; q < KL * NC / E; q += kThreads) {
      const int row = q / (NC / E), cc = E * (q % (NC / E));
      const int64_t gc = col0 + cc;
      const int64_t off = (r0 + row) * a.cols + gc;
      float f[E];
      if (a.vec && gc + E <= a.cols) {
        if constexpr (In::bytes == 4) {
          const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.src) + off);
          f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
        } else {
          const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src) + off);
          const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f[2 * j] = In::from_bits(static_cast<uint16_t>(w[j] & 0xFFFFu));
            f[2 * j + 1] = In::from_bits(static_cast<uint16_t>(w[j] >> 16));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) f[j] = (gc + j < a.cols) ? In::load(a.src, off + j) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < E; j += 4)
        *reinterpret_cast<float4*>(&tile[slot(row, cc + j)]) = make_float4(f[j], f[j + 1], f[j + 2], f[j + 3]);
    }
    __syncthreads();
    float v[M];
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] = tile[slot(p * M + i, c)];
    fwht_inreg<KL, M>(v);
#pragma unroll
    for (int m = 1; m < P; m <<= 1) fwht_xlane<M>(v, lane, m);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < M; ++i) tile[slot(p * M + i, c)] = v[i];
    __syncthreads();
    // eight consecutive columns per thread, written with 16-byte stores when whole and aligned
    for (int q = t; q < KL * NC / 8; q += kThreads) {
      const int row = q / (NC / 8), cc = 8 * (q % (NC / 8));
      const float4 x0 = *reinterpret_cast<const float4*>(&tile[slot(row, cc)]);
      const float4 x1 = *reinterpret_cast<const float4*>(&tile[slot(row, cc + 4)]);
      const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      if (a.nt)
        store_run<Out, 8, false, true>(a.dst, (r0 + row) * a.cols + col0 + cc, a.cols - (col0 + cc), f, 1.0f);
      else
        store_run<Out, 8>(a.dst, (r0 + row) * a.cols + col0 + cc, a.cols - (col0 + cc), f, 1.0f);
    }
  }
}

// ============================================================ register cols kernel (LEFT, k = 16)
// k = 16, 16-bit input, row pitch a multiple of 8 elements, 16-byte aligned source and
// destination. No LDS: a thread holds one whole 16-row block of 8 consecutive columns (one
// 16-byte load per row) and rotates it in registers; each load or store instruction covers
// 1 KB of one row. At 8192 x 13824 bf16 it runs in 83.5-86.2 us against 115-117 us for cols_kernel
// and 96.6 us on the matrix cores. The same layout at k = 32..256 (k/16 lanes per column group,
// the wider strides as DPP lane exchanges) was slower than cols_kernel at every such k (90.7,
// 100.2, 109.6, 135.1 against 85.1, 94.3, 103.0, 154.6 us; the matrix cores take 128 and 256),
// so it is built for k = 16 only.
constexpr int C16_COLS = 2048;   // columns per tile: 256 threads x 8
constexpr int kNt = 2;           // buffer-store cache policy: non-temporal
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <class In, class Out, bool NT>
__global__ __launch_bounds__(kThreads, 2) void cols16_kernel(ColArgs a) {
  if constexpr (In::bytes != 2) {
    return;
  } else {
    constexpr int R = 16;
    const int t = threadIdx.x;
    const int64_t nct = (a.cols + C16_COLS - 1) / C16_COLS;
    const int64_t tiles = (a.rows / R) * nct;
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
      const int64_t rb = (tile / nct) * R;
      const int64_t c0 = (tile % nct) * C16_COLS + 8 * t;
      if (c0 >= a.cols) continue;   // cols % 8 == 0: a thread's 8 columns are whole or absent
      // buffer loads and stores from the block's first row, the row index in the scalar offset
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(static_cast<const uint16_t*>(a.src) + rb * a.cols), 0,
          static_cast<int>(R * a.cols * 2), kBufferFlags);
      const int pitch = static_cast<int>(a.cols * 2);
      v4u x[R];
#pragma unroll
      for (int i = 0; i < R; ++i)
        x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(c0 * 2), i * pitch, 0);
      // two halves of four columns keep 64 values live; 16-bit outputs are packed into the input
      // words they replace, and a row leaves as one 16-byte store at the end
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float v[4 * R];   // (row i, column 4 hf + j) at v[4 i + j]
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t u = x[i][2 * hf + j];
            v[4 * i + 2 * j] = In::from_bits(static_cast<uint16_t>(u & 0xFFFFu));
            v[4 * i + 2 * j + 1] = In::from_bits(static_cast<uint16_t>(u >> 16));
          }
#pragma unroll
        for (int h = 1; h < R; h <<= 1)
#pragma unroll
          for (int i = 0; i < R; ++i)
            if ((i & h) == 0)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float p0 = v[4 * i + j], p1 = v[4 * (i + h) + j];
                v[4 * i + j] = p0 + p1;
                v[4 * (i + h) + j] = p0 - p1;
              }
        if constexpr (Out::bytes == 2) {
#pragma unroll
          for (int i = 0; i < R; ++i) {
            x[i][2 * hf] = Out::pack2(v[4 * i], v[4 * i + 1]);
            x[i][2 * hf + 1] = Out::pack2(v[4 * i + 2], v[4 * i + 3]);
          }
        } else {
          const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
              static_cast<float*>(a.dst) + rb * a.cols, 0, static_cast<int>(R * a.cols * 4), kBufferFlags);
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float4 f = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, f), rd,
                                                   static_cast<int>((c0 + 4 * hf) * 4), i * 2 * pitch,
                                                   NT ? kNt : 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one half's values live at a time
      }
      if constexpr (Out::bytes == 2) {
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<uint16_t*>(a.dst) + rb * a.cols, 0, static_cast<int>(R * a.cols * 2), kBufferFlags);
#pragma unroll
        for (int i = 0; i < R; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(x[i], rd, static_cast<int>(c0 * 2), i * pitch, NT ? kNt : 0);
      }
    }
  }
}

// ============================================================ fills
__global__ __launch_bounds__(kThreads) void zero_i32_kernel(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    p[i] = 0;
}

__global__ void write_scale_kernel(float* scale, const float* step) {
  *scale = step ? *step : 0.0f;
}

// ============================================================ launchers
static int grid_for(int64_t work, int per_block, int cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<int>(g);
}

template <class In, class Out>
static hipError_t launch_rows_k(int k, const RowArgs& a, int grid, hipStream_t st) {
  switch (k) {
#define HQ_ROWS_CASE(KK) \
  case KK: hipLaunchKernelGGL((rows_kernel<In, Out, KK>), dim3(grid), dim3(kThreads), 0, st, a); break;
    HQ_ROWS_CASE(1) HQ_ROWS_CASE(2) HQ_ROWS_CASE(4) HQ_ROWS_CASE(8) HQ_ROWS_CASE(16)
    HQ_ROWS_CASE(32) HQ_ROWS_CASE(64) HQ_ROWS_CASE(128) HQ_ROWS_CASE(256)
#undef HQ_ROWS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class In, class Out>
static hipError_t launch_cols_k(int k, const ColArgs& a, int grid, hipStream_t st) {
  switch (k) {
#define HQ_COLS_CASE(KK) \
  case KK: hipLaunchKernelGGL((cols_kernel<In, Out, KK>), dim3(grid), dim3(kThreads), 0, st, a); break;
    HQ_COLS_CASE(2) HQ_COLS_CASE(4) HQ_COLS_CASE(8) HQ_COLS_CASE(16)
    HQ_COLS_CASE(32) HQ_COLS_CASE(64) HQ_COLS_CASE(128) HQ_COLS_CASE(256)
#undef HQ_COLS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class In>
static hipError_t rows_out(int out_dt, int k, const RowArgs& a, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F32: return launch_rows_k<In, F32>(k, a, grid, st);
    case DT_F16: return launch_rows_k<In, F16>(k, a, grid, st);
    case DT_BF16: return launch_rows_k<In, BF16>(k, a, grid, st);
  }
  return hipErrorInvalidValue;
}

template <class In, bool NT>
static hipError_t cols16_out_nt(int out_dt, const ColArgs& a, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F32: hipLaunchKernelGGL((cols16_kernel<In, F32, NT>), dim3(grid), dim3(kThreads), 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL((cols16_kernel<In, F16, NT>), dim3(grid), dim3(kThreads), 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL((cols16_kernel<In, BF16, NT>), dim3(grid), dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class In>
static hipError_t cols16_out(int out_dt, const ColArgs& a, int grid, hipStream_t st) {
  return a.nt ? cols16_out_nt<In, true>(out_dt, a, grid, st) : cols16_out_nt<In, false>(out_dt, a, grid, st);
}

template <class In>
static hipError_t cols_out(int out_dt, int k, const ColArgs& a, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F32: return launch_cols_k<In, F32>(k, a, grid, st);
    case DT_F16: return launch_cols_k<In, F16>(k, a, grid, st);
    case DT_BF16: return launch_cols_k<In, BF16>(k, a, grid, st);
  }
  return hipErrorInvalidValue;
}

static int dt_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// hq_fwht writes its output once and reads nothing back: the stores carry the non-temporal
// hint unless HQ_FWHT_NT=0.
static int fwht_nt() {
  const char* e = std::getenv("HQ_FWHT_NT");
  return (e && e[0] == '0') ? 0 : 1;
}

hipError_t rows_pass(const RowPass& p, hipStream_t st) {
  RowArgs a{};
  a.src = p.src;
  a.rows = p.rows;
  a.cols = p.cols;
  a.vec = aligned16(p.src) && (p.cols * dt_bytes(p.in_dt)) % 16 == 0;
  a.dst = p.dst;
  // measured at 8192 x 13824 bf16: non-temporal stores take k >= 32 from 81-84 to 73-80 us,
  // but k = 16 (and the unrotated copy) from 82 to 94 us
  a.nt = p.k >= 32 ? fwht_nt() : 0;
  const int64_t lanes = p.rows * ((p.cols + 255) / 256) * 16;   // one 16-lane group per segment
  const int grid = grid_for(lanes, kThreads, 1 << 20);
  const int tok = prof_begin(K_ROT_STORE, static_cast<double>(p.rows) * p.cols *
                                              (dt_bytes(p.in_dt) + dt_bytes(p.out_dt)), st);
  hipError_t e = hipErrorInvalidValue;
  switch (p.in_dt) {
    case DT_F32: e = rows_out<F32>(p.out_dt, p.k, a, grid, st); break;
    case DT_F16: e = rows_out<F16>(p.out_dt, p.k, a, grid, st); break;
    case DT_BF16: e = rows_out<BF16>(p.out_dt, p.k, a, grid, st); break;
  }
  prof_end(tok, st);
  return e;
}

// At k = 16 the register kernel is the default where it applies; HQ_COLS_REG=0 selects the
// LDS-staged cols_kernel instead (read on every call, so the two can be measured side by side).
static bool cols_reg_on() {
  const char* e = std::getenv("HQ_COLS_REG");
  return !(e && e[0] == '0');
}

hipError_t cols_pass(const ColPass& p, hipStream_t st) {
  ColArgs a{};
  a.src = p.src;
  a.rows = p.rows;
  a.cols = p.cols;
  a.vec = aligned16(p.src) && (p.cols * dt_bytes(p.in_dt)) % 16 == 0;
  a.dst = p.dst;
  a.nt = fwht_nt();
  if ((p.in_dt == DT_F16 || p.in_dt == DT_BF16) && p.k == 16 && p.cols % 8 == 0 &&
      aligned16(p.src) && aligned16(p.dst) && 16 * p.cols * dt_bytes(p.out_dt) < (int64_t(1) << 31) &&
      cols_reg_on()) {
    const int64_t tiles = (p.rows / 16) * ((p.cols + C16_COLS - 1) / C16_COLS);
    const int tok = prof_begin(K_ROT_STORE, static_cast<double>(p.rows) * p.cols *
                                                (dt_bytes(p.in_dt) + dt_bytes(p.out_dt)), st);
    const int grid = grid_for(tiles, 1, 1 << 20);
    const hipError_t e = p.in_dt == DT_F16 ? cols16_out<F16>(p.out_dt, a, grid, st)
                                           : cols16_out<BF16>(p.out_dt, a, grid, st);
    prof_end(tok, st);
    return e;
  }
  const int nc = kThreads / (p.k >= 4 ? 4 : p.k);   // ColShape<k>::NC
  const int64_t tiles = (p.rows / p.k) * ((p.cols + nc - 1) / nc);
  const int grid = grid_for(tiles, 1, 1 << 20);
  const int tok = prof_begin(K_ROT_STORE, static_cast<double>(p.rows) * p.cols *
                                              (dt_bytes(p.in_dt) + dt_bytes(p.out_dt)), st);
  hipError_t e = hipErrorInvalidValue;
  switch (p.in_dt) {
    case DT_F32: e = cols_out<F32>(p.out_dt, p.k, a, grid, st); break;
    case DT_F16: e = cols_out<F16>(p.out_dt, p.k, a, grid, st); break;
    case DT_BF16: e = cols_out<BF16>(p.out_dt, p.k, a, grid, st); break;
  }
  prof_end(tok, st);
  return e;
}

hipError_t write_scale(float* scale, const float* step, hipStream_t st) {
  const int tok = prof_begin(K_MISC, 4.0, st);
  hipLaunchKernelGGL(write_scale_kernel, dim3(1), dim3(1), 0, st, scale, step);
  prof_end(tok, st);
  return hipGetLastError();
}

hipError_t zero_i32(int32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  const int grid = static_cast<int>(blocks < 1024 ? blocks : 1024);
  const int tok = prof_begin(K_MISC, 4.0 * n, st);
  hipLaunchKernelGGL(zero_i32_kernel, dim3(grid), dim3(kThreads), 0, st, p, n);
  prof_end(tok, st);
  return hipGetLastError();
}

}  // namespace hq
