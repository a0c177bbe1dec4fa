// hq_rotate.hip — block-diagonal Walsh-Hadamard rotation, tensor-wise absmax and
// round-to-nearest quantization kernels for gfx950.
//
// "Training Transformers with 4-bit Integers", §3.3 (block-diagonal H_k transform spreads
// outliers before quantization), §3.1 (quantizer onto a symmetric integer grid) and §A.6
// (Hadamard multiplication, quantization and packing precede the integer GEMM);
// "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs", Approach (right rotation of
// X and W, left / token-axis rotation of dY, one scale per tensor).
//
// Two transform shapes:
//   rows kernel  — rotation along the contiguous axis (RIGHT). A 16-lane group owns a 256-column
//                  segment of one row; each lane owns 16 consecutive elements, so strides < 16
//                  are in-register butterflies and strides 16..128 are lane exchanges.
//   cols kernel  — rotation along the row axis (LEFT, the token axis). A workgroup stages a
//                  KL-row tile in LDS (fp32, column-swizzled), each thread owns KL/P consecutive
//                  rows of one column (in-register stages) and P lanes share a column.
// Each runs as an absmax pass (one partial max per workgroup, no atomics, so the result is
// order-independent), a quantize pass (reads the partials, writes codes and the scale), or a
// store pass (writes the rotated values in a floating-point dtype).
#include "hq_device.hpp"
#include "hq_internal.hpp"

namespace hq {

constexpr int kThreads = 256;

// ============================================================ rows kernel (RIGHT / NONE)
struct RowArgs {
  const void* src;
  int64_t rows, cols;   // src is rows x cols, row pitch = cols elements
  bool vec;             // 16-byte loads are legal for every full 16-element chunk
  int op;               // OP_ABSMAX / OP_QUANT / OP_STORE
  float* partials;      // ABSMAX out: one per workgroup
  const float* part_in; // QUANT in
  int nparts;
  const float* step;    // QUANT: STEP mode (else nullptr)
  int qp;
  float* scale_out;     // QUANT: written by workgroup 0
  int8_t* codes;        // QUANT: rows x cols codes, pitch ld
  int64_t ld;
  void* dst;            // STORE: rows x cols output (pitch cols)
};

template <class In, class Out, int KR, int OP>
__global__ __launch_bounds__(kThreads) void rows_kernel(RowArgs a) {
  __shared__ float red[32];
  const int lane = threadIdx.x & 63;
  const int g = lane & 15;                        // lane within the 16-lane group
  const int group = (blockIdx.x * kThreads + threadIdx.x) >> 4;
  const int ngroups = (gridDim.x * kThreads) >> 4;
  const int64_t nseg = (a.cols + 255) / 256;
  const int64_t items = a.rows * nseg;

  float s = 0.0f, r = 0.0f;
  if constexpr (OP == OP_QUANT) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qp, red, s, r);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.scale_out = s;
  }
  float amax = 0.0f;

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
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    } else if constexpr (OP == OP_QUANT) {
      // columns >= cols hold zeros, so the 16-byte chunk also zero-fills the pitch padding
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack4(quant_code(v[4 * q], r, a.qp), quant_code(v[4 * q + 1], r, a.qp),
                     quant_code(v[4 * q + 2], r, a.qp), quant_code(v[4 * q + 3], r, a.qp));
      *reinterpret_cast<uint4*>(a.codes + row * a.ld + c0) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      const int64_t base = row * a.cols;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (c0 + j < a.cols) Out::store(a.dst, base + c0 + j, v[j]);
    }
  }
  if constexpr (OP == OP_ABSMAX) {
    amax = block_max(amax, red);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = amax;
  }
}

// ============================================================ cols kernel (LEFT)
struct ColArgs {
  const void* src;
  int64_t rows, cols;   // rows % KL == 0
  bool vec;             // 4-element loads are aligned (cols % 4 == 0 and base aligned)
  int op;
  float* partials;
  const float* part_in;
  int nparts;
  const float* step;
  int qp;
  float* scale_out;
  int8_t* codes_t;      // QUANT: cols x rows codes (transposed), pitch ld_t
  int64_t ld_t;
  void* dst;            // STORE: rows x cols output
};

template <int KL> struct ColShape {
  static constexpr int P = KL >= 4 ? 4 : KL;      // lanes sharing one column
  static constexpr int M = KL / P;                // rows per thread
  static constexpr int NC = kThreads / P;         // columns per tile
};

template <class In, class Out, int KL, int OP>
__global__ __launch_bounds__(kThreads) void cols_kernel(ColArgs a) {
  using S = ColShape<KL>;
  constexpr int P = S::P, M = S::M, NC = S::NC;
  __shared__ float tile[KL * NC];
  __shared__ float red[32];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int c = t / P, p = t % P;
  const int64_t nrb = a.rows / KL;
  const int64_t ncb = (a.cols + NC - 1) / NC;
  const int64_t tiles = nrb * ncb;

  float s = 0.0f, r = 0.0f;
  if constexpr (OP == OP_QUANT) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qp, red, s, r);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.scale_out = s;
  }
  float amax = 0.0f;
  // element (row, col) of the tile lives at row*NC + (col ^ (16 * (row / M)))
  auto slot = [](int row, int col) { return row * NC + (col ^ (16 * (row / M))); };

  for (int64_t tile_id = blockIdx.x; tile_id < tiles; tile_id += gridDim.x) {
    const int64_t r0 = (tile_id / ncb) * KL;
    const int64_t col0 = (tile_id % ncb) * NC;
    __syncthreads();
    // stage KL x NC values, 4 consecutive columns per thread per step
    for (int q = t; q < KL * NC / 4; q += kThreads) {
      const int row = q / (NC / 4), cc = 4 * (q % (NC / 4));
      const int64_t gc = col0 + cc;
      const int64_t off = (r0 + row) * a.cols + gc;
      float f[4];
      if (a.vec && gc + 4 <= a.cols) {
        if constexpr (In::bytes == 4) {
          float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.src) + off);
          f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
        } else {
          uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.src) + off);
          f[0] = In::from_bits(x.x & 0xFFFFu); f[1] = In::from_bits(x.x >> 16);
          f[2] = In::from_bits(x.y & 0xFFFFu); f[3] = In::from_bits(x.y >> 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = (gc + j < a.cols) ? In::load(a.src, off + j) : 0.0f;
      }
      *reinterpret_cast<float4*>(&tile[slot(row, cc)]) = make_float4(f[0], f[1], f[2], f[3]);
    }
    __syncthreads();
    float v[M];
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] = tile[slot(p * M + i, c)];
    fwht_inreg<KL, M>(v);
#pragma unroll
    for (int m = 1; m < P; m <<= 1) fwht_xlane<M>(v, lane, m);

    const int64_t gcol = col0 + c;
    if constexpr (OP == OP_ABSMAX) {
      if (gcol < a.cols) {
#pragma unroll
        for (int i = 0; i < M; ++i) amax = fmaxf(amax, fabsf(v[i]));
      }
    } else if constexpr (OP == OP_QUANT) {
      if (gcol < a.cols) {
        int8_t* dst = a.codes_t + gcol * a.ld_t + r0 + p * M;
        if constexpr (M % 16 == 0) {
#pragma unroll
          for (int q = 0; q < M / 16; ++q) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              w[j] = pack4(quant_code(v[16 * q + 4 * j], r, a.qp),
                           quant_code(v[16 * q + 4 * j + 1], r, a.qp),
                           quant_code(v[16 * q + 4 * j + 2], r, a.qp),
                           quant_code(v[16 * q + 4 * j + 3], r, a.qp));
            *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(w[0], w[1], w[2], w[3]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < M; ++i) dst[i] = static_cast<int8_t>(quant_code(v[i], r, a.qp));
        }
      }
    } else {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < M; ++i) tile[slot(p * M + i, c)] = v[i];
      __syncthreads();
      for (int q = t; q < KL * NC / 4; q += kThreads) {
        const int row = q / (NC / 4), cc = 4 * (q % (NC / 4));
        const float4 x = *reinterpret_cast<const float4*>(&tile[slot(row, cc)]);
        const float f[4] = {x.x, x.y, x.z, x.w};
        const int64_t off = (r0 + row) * a.cols + col0 + cc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col0 + cc + j < a.cols) Out::store(a.dst, off + j, f[j]);
      }
    }
  }
  if constexpr (OP == OP_ABSMAX) {
    amax = block_max(amax, red);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = amax;
  }
}

// ============================================================ int8 transpose
// dst (cols x rows, pitch ld_dst) = src^T (src rows x cols, pitch ld_src); zero-fills the
// dst pitch padding up to the next multiple of 16 after `rows`.
__global__ __launch_bounds__(kThreads) void transpose_i8_kernel(const int8_t* src, int64_t ld_src,
                                                                int8_t* dst, int64_t ld_dst,
                                                                int64_t rows, int64_t cols) {
  __shared__ int8_t tile[64][64 + 4];
  const int64_t rpad = (rows + 15) / 16 * 16;
  const int64_t nrt = (rpad + 63) / 64, nct = (cols + 63) / 64;
  for (int64_t tid = blockIdx.x; tid < nrt * nct; tid += gridDim.x) {
    const int64_t r0 = (tid / nct) * 64, c0 = (tid % nct) * 64;
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * 64; q += kThreads) {
      const int i = q / 64, j = q % 64;
      const int64_t gr = r0 + i, gc = c0 + j;
      tile[i][j] = (gr < rows && gc < cols) ? src[gr * ld_src + gc] : int8_t(0);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * 64; q += kThreads) {
      const int j = q / 64, i = q % 64;   // dst row j (src column), dst column i (src row)
      const int64_t gc = c0 + j, gr = r0 + i;
      if (gc < cols && gr < rpad) dst[gc * ld_dst + gr] = tile[i][j];
    }
  }
}

// Zero bytes [from, to) of each of nrows rows of pitch ld.
__global__ __launch_bounds__(kThreads) void zero_pad_kernel(int8_t* p, int64_t nrows, int64_t ld,
                                                            int64_t from, int64_t to) {
  const int64_t w = to - from;
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nrows * w;
       i += (int64_t)gridDim.x * kThreads)
    p[(i / w) * ld + from + i % w] = 0;
}

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

template <class In, class Out, int OP>
static hipError_t launch_rows_k(int k, const RowArgs& a, int grid, hipStream_t st) {
  switch (k) {
#define HQ_ROWS_CASE(KK) \
  case KK: hipLaunchKernelGGL((rows_kernel<In, Out, KK, OP>), dim3(grid), dim3(kThreads), 0, st, a); break;
    HQ_ROWS_CASE(1) HQ_ROWS_CASE(2) HQ_ROWS_CASE(4) HQ_ROWS_CASE(8) HQ_ROWS_CASE(16)
    HQ_ROWS_CASE(32) HQ_ROWS_CASE(64) HQ_ROWS_CASE(128) HQ_ROWS_CASE(256)
#undef HQ_ROWS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class In, class Out, int OP>
static hipError_t launch_cols_k(int k, const ColArgs& a, int grid, hipStream_t st) {
  switch (k) {
#define HQ_COLS_CASE(KK) \
  case KK: hipLaunchKernelGGL((cols_kernel<In, Out, KK, OP>), dim3(grid), dim3(kThreads), 0, st, a); break;
    HQ_COLS_CASE(2) HQ_COLS_CASE(4) HQ_COLS_CASE(8) HQ_COLS_CASE(16)
    HQ_COLS_CASE(32) HQ_COLS_CASE(64) HQ_COLS_CASE(128) HQ_COLS_CASE(256)
#undef HQ_COLS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class In, int OP>
static hipError_t dispatch_rows_out(int out_dt, int k, const RowArgs& a, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F32: return launch_rows_k<In, F32, OP>(k, a, grid, st);
    case DT_F16: return launch_rows_k<In, F16, OP>(k, a, grid, st);
    case DT_BF16: return launch_rows_k<In, BF16, OP>(k, a, grid, st);
  }
  return hipErrorInvalidValue;
}

template <class In, int OP>
static hipError_t dispatch_cols_out(int out_dt, int k, const ColArgs& a, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F32: return launch_cols_k<In, F32, OP>(k, a, grid, st);
    case DT_F16: return launch_cols_k<In, F16, OP>(k, a, grid, st);
    case DT_BF16: return launch_cols_k<In, BF16, OP>(k, a, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int OP>
static hipError_t dispatch_rows(int in_dt, int out_dt, int k, const RowArgs& a, int grid,
                                hipStream_t st) {
  switch (in_dt) {
    case DT_F32: return dispatch_rows_out<F32, OP>(out_dt, k, a, grid, st);
    case DT_F16: return dispatch_rows_out<F16, OP>(out_dt, k, a, grid, st);
    case DT_BF16: return dispatch_rows_out<BF16, OP>(out_dt, k, a, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int OP>
static hipError_t dispatch_cols(int in_dt, int out_dt, int k, const ColArgs& a, int grid,
                                hipStream_t st) {
  switch (in_dt) {
    case DT_F32: return dispatch_cols_out<F32, OP>(out_dt, k, a, grid, st);
    case DT_F16: return dispatch_cols_out<F16, OP>(out_dt, k, a, grid, st);
    case DT_BF16: return dispatch_cols_out<BF16, OP>(out_dt, k, a, grid, st);
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
  a.op = p.op;
  a.partials = p.partials;
  a.part_in = p.part_in;
  a.nparts = p.nparts;
  a.step = p.step;
  a.qp = p.qp;
  a.scale_out = p.scale_out;
  a.codes = p.codes;
  a.ld = p.ld;
  a.dst = p.dst;
  const int64_t items = p.rows * ((p.cols + 255) / 256) * 16;   // lanes of work
  int grid = (p.op == OP_ABSMAX) ? grid_for(items, kThreads, kMaxPartials)
                                 : grid_for(items, kThreads, 1 << 20);
  const double in_b = static_cast<double>(p.rows) * p.cols * dt_bytes(p.in_dt);
  hipError_t e = hipErrorInvalidValue;
  int tok;
  switch (p.op) {
    case OP_ABSMAX:
      tok = prof_begin(K_ROT_ABSMAX, in_b, st);
      e = dispatch_rows<OP_ABSMAX>(p.in_dt, DT_F32, p.k, a, grid, st);
      break;
    case OP_QUANT:
      tok = prof_begin(K_ROT_QUANT, in_b + static_cast<double>(p.rows) * p.cols, st);
      e = dispatch_rows<OP_QUANT>(p.in_dt, DT_F32, p.k, a, grid, st);
      break;
    default:
      tok = prof_begin(K_ROT_STORE, in_b + static_cast<double>(p.rows) * p.cols * dt_bytes(p.out_dt), st);
      e = dispatch_rows<OP_STORE>(p.in_dt, p.out_dt, p.k, a, grid, st);
      break;
  }
  prof_end(tok, st);
  return e;
}

int rows_pass_grid(const RowPass& p) {
  const int64_t items = p.rows * ((p.cols + 255) / 256) * 16;
  return grid_for(items, kThreads, kMaxPartials);
}

static int cols_tile_cols(int k) { return kThreads / (k >= 4 ? 4 : k); }

hipError_t cols_pass(const ColPass& p, hipStream_t st) {
  ColArgs a{};
  a.src = p.src;
  a.rows = p.rows;
  a.cols = p.cols;
  a.vec = aligned16(p.src) && (p.cols % 4) == 0;
  a.op = p.op;
  a.partials = p.partials;
  a.part_in = p.part_in;
  a.nparts = p.nparts;
  a.step = p.step;
  a.qp = p.qp;
  a.scale_out = p.scale_out;
  a.codes_t = p.codes_t;
  a.ld_t = p.ld_t;
  a.dst = p.dst;
  const int nc = cols_tile_cols(p.k);
  const int64_t tiles = (p.rows / p.k) * ((p.cols + nc - 1) / nc);
  int grid = (p.op == OP_ABSMAX) ? grid_for(tiles, 1, kMaxPartials) : grid_for(tiles, 1, 1 << 20);
  const double in_b = static_cast<double>(p.rows) * p.cols * dt_bytes(p.in_dt);
  hipError_t e = hipErrorInvalidValue;
  int tok;
  switch (p.op) {
    case OP_ABSMAX:
      tok = prof_begin(K_ROT_ABSMAX, in_b, st);
      e = dispatch_cols<OP_ABSMAX>(p.in_dt, DT_F32, p.k, a, grid, st);
      break;
    case OP_QUANT:
      tok = prof_begin(K_ROT_QUANT, in_b + static_cast<double>(p.rows) * p.cols, st);
      e = dispatch_cols<OP_QUANT>(p.in_dt, DT_F32, p.k, a, grid, st);
      break;
    default:
      tok = prof_begin(K_ROT_STORE, in_b + static_cast<double>(p.rows) * p.cols * dt_bytes(p.out_dt), st);
      e = dispatch_cols<OP_STORE>(p.in_dt, p.out_dt, p.k, a, grid, st);
      break;
  }
  prof_end(tok, st);
  return e;
}

int cols_pass_grid(const ColPass& p) {
  const int nc = cols_tile_cols(p.k);
  const int64_t tiles = (p.rows / p.k) * ((p.cols + nc - 1) / nc);
  return grid_for(tiles, 1, kMaxPartials);
}

hipError_t transpose_i8(const int8_t* src, int64_t ld_src, int8_t* dst, int64_t ld_dst,
                        int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t rpad = (rows + 15) / 16 * 16;
  const int64_t tiles = ((rpad + 63) / 64) * ((cols + 63) / 64);
  if (tiles == 0) return hipSuccess;
  const int grid = grid_for(tiles, 1, 1 << 20);
  const int tok = prof_begin(K_TRANSPOSE, 2.0 * rows * cols, st);
  hipLaunchKernelGGL(transpose_i8_kernel, dim3(grid), dim3(kThreads), 0, st, src, ld_src, dst,
                     ld_dst, rows, cols);
  prof_end(tok, st);
  return hipGetLastError();
}

hipError_t zero_pad(int8_t* p, int64_t nrows, int64_t ld, int64_t from, int64_t to,
                    hipStream_t st) {
  if (to <= from || nrows == 0) return hipSuccess;
  const int grid = grid_for(nrows * (to - from), kThreads, 4096);
  const int tok = prof_begin(K_MISC, static_cast<double>(nrows) * (to - from), st);
  hipLaunchKernelGGL(zero_pad_kernel, dim3(grid), dim3(kThreads), 0, st, p, nrows, ld, from, to);
  prof_end(tok, st);
  return hipGetLastError();
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
