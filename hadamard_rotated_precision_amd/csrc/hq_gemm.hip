// hq_gemm.hip — INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores, with a fused dequantizing
// epilogue ("Training Transformers with 4-bit Integers", §3.1: the integer product is
// accumulated in INT32 and dequantized back to floating point; §A.6: the integer GEMM reads
// both operands contiguous along K).
//
// c[m][n] = sum_k a[m][k] * b[n][k]; a is M x K and b is N x K, both K-contiguous int8.
// Design for CDNA4:
//   - 256 x 256 output tile per workgroup, 4 wave64s in a 2 x 2 grid, 128 x 128 per wave built
//     from 4 x 4 blocks of v_mfma_i32_32x32x32_i8 (int32 accumulators, 256 per lane);
//   - K advances 64 bytes per step through a double-buffered LDS stage (2 x 32 KB); global
//     loads for step t+1 are issued before the MFMAs of step t;
//   - LDS rows are 64 bytes; the 16-byte chunk index is XOR-swizzled with (row / 4) % 4 so the
//     128-bit fragment reads of 16 consecutive rows hit 16 distinct bank groups;
//   - workgroups are remapped so that consecutive tiles of a group land on one XCD (blocks are
//     dispatched round-robin over the 8 XCDs) and tiles of a group share A rows in its L2.
#include "hq_device.hpp"
#include "hq_internal.hpp"

namespace hq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;

struct GemmArgs {
  const int8_t* a;
  int64_t lda;
  const int8_t* b;
  int64_t ldb;
  int64_t M, N, K;
  void* c;
  int64_t ldc;
  const float* sa;
  const float* sb;
  float kmul;
};

__device__ inline int lds_off(int row, int chunk) {
  return row * GBK + ((chunk ^ ((row >> 2) & 3)) << 4);
}

template <class Out, int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_i8_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2][(GBM + GBN) * GBK];

  const int tiles_m = static_cast<int>((g.M + GBM - 1) / GBM);
  const int tiles_n = static_cast<int>((g.N + GBN - 1) / GBN);
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);   // XCD-contiguous
  const int group = pid / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (pid % (kGroupM * tiles_n)) % gsize;
  const int tn = (pid % (kGroupM * tiles_n)) / gsize;
  const int64_t m0 = static_cast<int64_t>(tm) * GBM, n0 = static_cast<int64_t>(tn) * GBN;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int KT = static_cast<int>((g.K + GBK - 1) / GBK);
  v4i stage[8];

  auto load_tile = [&](int kt) {
    const int64_t k0 = static_cast<int64_t>(kt) * GBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = t + kGemmThreads * j;
      const int row = q >> 2, ch = q & 3;
      const int64_t kk = k0 + 16 * ch;
      const int64_t ga = m0 + row, gb = n0 + row;
      v4i za = {0, 0, 0, 0}, zb = {0, 0, 0, 0};
      if (ga < g.M && kk < g.K) za = *reinterpret_cast<const v4i*>(g.a + ga * g.lda + kk);
      if (gb < g.N && kk < g.K) zb = *reinterpret_cast<const v4i*>(g.b + gb * g.ldb + kk);
      stage[j] = za;
      stage[4 + j] = zb;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = t + kGemmThreads * j;
      const int row = q >> 2, ch = q & 3;
      *reinterpret_cast<v4i*>(&smem[buf][lds_off(row, ch)]) = stage[j];
      *reinterpret_cast<v4i*>(&smem[buf][GBM * GBK + lds_off(row, ch)]) = stage[4 + j];
    }
  };

  if (KT > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    const int8_t* sa = smem[cur];
    const int8_t* sb = smem[cur] + GBM * GBK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const v4i*>(sa + lds_off(row, ch));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const v4i*>(sb + lds_off(row, ch));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue. 32x32 accumulator layout: lane holds column (lane % 32) and, in register r,
  // row 8*(r/4) + 4*(lane/32) + r%4 of its block.
  float alpha = 1.0f;
  if constexpr (EPI == EPI_SCALE) alpha = (*g.sa * *g.sb) * g.kmul;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < g.M && col < g.N) {
          if constexpr (EPI == EPI_I32) {
            static_cast<int32_t*>(g.c)[row * g.ldc + col] = acc[i][j][r];
          } else {
            Out::store(g.c, row * g.ldc + col, static_cast<float>(acc[i][j][r]) * alpha);
          }
        }
      }
    }
}

template <class Out, int EPI>
static hipError_t launch_gemm(const GemmArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_i8_kernel<Out, EPI>), dim3(grid), dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t gemm_pass(const GemmPass& p, hipStream_t st) {
  GemmArgs a{p.a, p.lda, p.b, p.ldb, p.M, p.N, p.K, p.c, p.ldc, p.sa, p.sb, p.kmul};
  const int64_t tiles = ((p.M + GBM - 1) / GBM) * ((p.N + GBN - 1) / GBN);
  if (tiles == 0) return hipSuccess;
  const int grid = static_cast<int>(tiles);
  if (p.epi == EPI_I32) return launch_gemm<F32, EPI_I32>(a, grid, st);
  switch (p.out_dt) {
    case DT_F32: return launch_gemm<F32, EPI_SCALE>(a, grid, st);
    case DT_F16: return launch_gemm<F16, EPI_SCALE>(a, grid, st);
    case DT_BF16: return launch_gemm<BF16, EPI_SCALE>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hq
