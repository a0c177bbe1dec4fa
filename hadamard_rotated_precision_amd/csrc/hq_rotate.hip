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
#include "hq_device.hpp"
#include "hq_internal.hpp"

namespace hq {

constexpr int kThreads = 256;

// ============================================================ rows kernel (RIGHT / NONE)
struct RowArgs {
  const void* src;
  int64_t rows, cols;   // src is rows x cols, row pitch = cols elements
  bool vec;             // 16-byte loads are legal for every full 16-element chunk
  void* dst;            // rows x cols output (pitch cols)
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
    store_run<Out, 16>(a.dst, row * a.cols + c0, a.cols - c0, v, 1.0f);
  }
}

// ============================================================ cols kernel (LEFT)
struct ColArgs {
  const void* src;
  int64_t rows, cols;   // rows % KL == 0
  bool vec;             // 16-byte loads are aligned (row pitch a multiple of 16 bytes, base aligned)
  void* dst;            // rows x cols output
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
      store_run<Out, 8>(a.dst, (r0 + row) * a.cols + col0 + cc, a.cols - (col0 + cc), f, 1.0f);
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

hipError_t rows_pass(const RowPass& p, hipStream_t st) {
  RowArgs a{};
  a.src = p.src;
  a.rows = p.rows;
  a.cols = p.cols;
  a.vec = aligned16(p.src) && (p.cols * dt_bytes(p.in_dt)) % 16 == 0;
  a.dst = p.dst;
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

hipError_t cols_pass(const ColPass& p, hipStream_t st) {
  ColArgs a{};
  a.src = p.src;
  a.rows = p.rows;
  a.cols = p.cols;
  a.vec = aligned16(p.src) && (p.cols * dt_bytes(p.in_dt)) % 16 == 0;
  a.dst = p.dst;
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
