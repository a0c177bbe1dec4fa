// hq_gemm.hip — INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores with a fused epilogue that
// dequantizes, applies the output-side inverse Walsh-Hadamard rotations and stores. The same
// kernel also multiplies FP8 (OCP E4M3) codes with fp32 accumulation (F8: the HALO page's FP8
// variant of the three matmuls): v_mfma_f32_32x32x64_f8f6f4 takes 32 K bytes per lane; a lane
// reads the same two 16-byte chunks of its A row and of its B row, so the products the
// instruction pairs up share their K index whatever its internal byte order.
//
// "Training Transformers with 4-bit Integers", §3.1 (integer product accumulated in INT32,
// dequantized back to floating point), §3.3 (the block-diagonal H_k transforms cancel, so the
// output side multiplies by H_k once more per rotated axis), §A.6 (HQ-MM stages; the integer
// GEMM reads both operands contiguous along K).
//
// c[m][n] = sum_k a[m][k] * b[n][k];  a: M x K, b: N x K, int8, K-contiguous.
//
// Main loop (CDNA4):
//   - workgroup tile 256 x BN (BN = 256 or 128) from eight wave64s of 128 x BN/4 in a 2 x 4
//     grid, two waves per SIMD; a wave holds 4 x BN/128 v_mfma_i32_32x32x32_i8 tiles (128 or 64
//     int32 accumulators in AGPRs), so one wave's LDS and memory waits are covered by the other
//     wave's MFMAs;
//   - K advances 128 bytes per step. Operands go from memory straight into LDS (buffer loads
//     with the lds bit): two 64 KB stages for 256-wide tiles (loads one step ahead), three
//     48 KB stages for 128-wide ones (two steps ahead). One barrier per step; the first
//     fragments of the next step are read right after it, before the current step's last
//     MFMAs, so the matrix pipe keeps busy across it;
//   - LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with (row / 2) % 8 so the
//     128-bit fragment reads of 16 consecutive rows cover the 64 banks once;
//   - workgroups are remapped so consecutive tiles land on one XCD (blocks are dispatched
//     round-robin over the 8 XCDs) and a group of tiles shares A rows in that XCD's L2.
//
// Epilogue (EPI_SCALE): acc -> fp32, then
//   - rotation along M (rows) in registers: in the 32x32 accumulator layout a lane holds 16 rows
//     of each of its 4 row blocks, so row bits 0,1,3,4 (register index) and 5,6 (block index) are
//     in-lane butterflies, bit 2 is the lane half (v_permlane32_swap), bit 7 is the wave row
//     (done in the LDS phase below);
//   - the tile is staged through LDS in rounds that hold the same rows of both wave rows (rows
//     x and x+128 of the tile together, so the bit-7 butterfly is local): four rounds of 2 x 32
//     rows, two of 2 x 64 in TRANS mode. There the column rotation (along N) and the cast to the
//     output dtype happen in a row-contiguous thread layout, and stores are coalesced; TRANS
//     mode stores the transpose (the caller computes the transposed product when only the
//     rows need rotating, which keeps that rotation in registers).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "hq_device.hpp"
#include "hq_internal.hpp"
#include "hq_launch.hpp"

namespace hq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int GBM = 256;
constexpr int kGroupM = 8;
constexpr int kOutOfRange = 0x7FFFFFF0;    // an offset past any descriptor: the load reads 0

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
  float* pair_part;      // PAIR: 2 fp32 partial tiles per pair of 256 x 128 tiles
  int32_t* pair_cnt;     // PAIR: arrival flags per pair (zero on entry, left set)
  int pair_spin;         // PAIR: polls of the partner's flag before the wait-free fallback
  // batched products (grid.y = batch index): offsets of a batch's a and b (bytes) and c
  // (elements); the scales are shared (one per batched tensor)
  int64_t a_bstride, b_bstride, c_bstride;
  // when set, the contraction stops at min(K, *k_dev) (a length an earlier kernel on the stream
  // wrote, e.g. the number of sampled rows); operand bytes from there to the next multiple of
  // 16 must be zero
  const int32_t* k_dev;
  int nt;                // EPI_SCALE: outputs stored with the non-temporal hint (default)
};


// LDS layout of an operand stage: rows of KB bytes (KB = K bytes per step), the 16-byte chunk
// index XOR-swizzled so that the 128-bit fragment reads of 16 consecutive rows hit 16
// distinct 16-byte bank groups.
template <int KB>
__device__ inline int lds_off(int row, int chunk) {
  const int swz = (KB == 64) ? ((row >> 2) & 3) : ((row >> 1) & 7);
  return row * KB + ((chunk ^ swz) << 4);
}

// In-register butterflies along the tile's M axis for row bits 0,1,3,4 (register index) and
// 5,6 (row-block index), restricted to strides < KM. v[bi][bj][r]: row = 32*bi + 8*(r/4) +
// 4*(lane/32) + r%4 within the wave's 128 rows.
template <int KM, int NB, class V>
__device__ inline void rows_fwht_inlane(V (&v)[4][NB]) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
      // row strides 1, 2 <- register bits 0, 1; row strides 8, 16 <- register bits 2, 3
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int stride = (rb < 2) ? (1 << rb) : (8 << (rb - 2));
        if (stride < KM) {
          const int h = 1 << rb;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((r & h) == 0) {
              float a = v[bi][bj][r], b = v[bi][bj][r + h];
              v[bi][bj][r] = a + b;
              v[bi][bj][r + h] = a - b;
            }
        }
      }
    }
  // row strides 32, 64 <- block bits 0, 1
#pragma unroll
  for (int hb = 1; hb <= 2; hb <<= 1) {
    if (32 * hb < KM) {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        if ((bi & hb) == 0)
#pragma unroll
          for (int bj = 0; bj < NB; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float a = v[bi][bj][r], b = v[bi + hb][bj][r];
              v[bi][bj][r] = a + b;
              v[bi + hb][bj][r] = a - b;
            }
    }
  }
}

// Row stride 4 <- lane bit 5: the pair lives in lanes l and l^32. One row block (the stage
// pairs values within a block, so the row-major epilogue applies it block by block, which
// keeps the swap results of one block, not of all four, in registers at a time).
// Two values a, b per step: a swap of a's upper half with b's lower half leaves the lower lanes
// holding both halves of a and the upper lanes both halves of b; each lane forms the sum and
// the difference of its pair, and a second swap returns sums to the lower lanes and
// differences to the upper ones, each value in its own register again (two swaps and two
// adds for two values).
template <int NB, class V>
__device__ inline void rows_fwht_lanehalf_block(V (&v)[NB], int lane) {
#pragma unroll
  for (int bj = 0; bj < NB; ++bj)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[bj][r]),
                                                __float_as_uint(v[bj][r + 1]), false, false);
      const float lo = __uint_as_float(p[0]), hi = __uint_as_float(p[1]);
      auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo + hi), __float_as_uint(lo - hi),
                                                false, false);
      v[bj][r] = __uint_as_float(q[0]);       // lower lane: a_lo + a_hi, upper: a_lo - a_hi
      v[bj][r + 1] = __uint_as_float(q[1]);   // the same for b
    }
}

template <int NB, class V>
__device__ inline void rows_fwht_lanehalf(V (&v)[4][NB], int lane) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) rows_fwht_lanehalf_block<NB>(v[bi], lane);
}

// Butterfly stages over lanes l ^ m (m = 1, 2, 4) for N values.
template <int N>
__device__ inline void xlane_stage(float (&v)[N], int lane, int m) {
  const bool upper = (lane & m) != 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float p = __shfl_xor(v[i], m, 64);
    v[i] = upper ? (p - v[i]) : (v[i] + p);
  }
}

// Threads of a workgroup for a 256 x BN tile: eight waves of 128 x WN in a 2 x (BN/WN) grid
// (WN = 64 for 256-wide tiles, 32 for 128-wide ones), two waves per SIMD.
template <int BN> struct GemmShape {
  static constexpr int WN = BN == 256 ? 64 : 32;
  static constexpr int NW = 2 * (BN / WN);
  static constexpr int NT = 64 * NW;
};

template <int BN, class Out, int EPI, int KM, int KN, bool TRANS, bool PAIR, bool F8>
__global__ __launch_bounds__(GemmShape<BN>::NT, 1) void gemm_i8_kernel(GemmArgs g) {
  if (blockIdx.y > 0) {   // batch blockIdx.y of a batched product (never with tile pairs)
    g.a += blockIdx.y * g.a_bstride;
    g.b += blockIdx.y * g.b_bstride;
    const size_t esz = (EPI == EPI_I32) ? 4 : Out::bytes;
    g.c = static_cast<char*>(g.c) + static_cast<size_t>(blockIdx.y) * g.c_bstride * esz;
  }
  constexpr int NT = GemmShape<BN>::NT;   // 512: two waves per SIMD
  constexpr int NW = GemmShape<BN>::NW;
  constexpr int WN = GemmShape<BN>::WN;   // wave tile columns
  constexpr int NB = WN / 32;         // 32x32 blocks per wave along N
  constexpr int WCOLS = BN / WN;      // waves along N
  // K bytes per step and LDS stages: 128 bytes in two 64 KB stages for 256-wide tiles, in
  // three 48 KB stages for 128-wide ones (one barrier per 32 or 16 MFMAs per wave)
  constexpr int GBK = 128;
  constexpr int NST = BN == 256 ? 2 : 3;
  // K slices per step, one MFMA group each: 32 bytes (int8) or 64 bytes (FP8)
  constexpr int KS = F8 ? GBK / 64 : GBK / 32;
  constexpr int KC = GBK / 16;        // 16-byte chunks per LDS row
  constexpr int RPB = 1024 / GBK;     // rows per 1 KB direct-to-LDS block
  constexpr int A_BYTES = GBM * GBK, B_BYTES = BN * GBK, STAGE = A_BYTES + B_BYTES;
  // LDS stages, each its own LDS object so the compiler tracks which direct-to-LDS loads a
  // fragment read has to wait for; the epilogue reuses stages 0 and 1 (64 rows x BN fp32 each).
  constexpr int STAGE_ALLOC = STAGE;
  static_assert(64 * BN * 4 <= STAGE, "an epilogue round must fit one stage");
  __shared__ __attribute__((aligned(16))) int8_t st0[STAGE_ALLOC];
  __shared__ __attribute__((aligned(16))) int8_t st1[STAGE_ALLOC];
  __shared__ __attribute__((aligned(16))) int8_t st2[NST == 3 ? STAGE_ALLOC : 16];
  // The row-major epilogue with 128- or 256-point row rotations on 256-wide tiles parks the last
  // round's block of values in LDS while the first rounds run (see STASH below); two of its
  // eight 16-byte chunks per thread live here, the rest in the unused tails of stages 0 and 1.
  constexpr bool STASH = BN == 256 && !TRANS && !PAIR && KM >= 128 && EPI != EPI_I32;
  __shared__ __attribute__((aligned(16))) float4 stash_x[STASH ? 2 * NT : 1];

  const int tiles_m = static_cast<int>((g.M + GBM - 1) / GBM);
  const int tiles_n = static_cast<int>((g.N + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  // XCD-contiguous order: block b runs on XCD b % 8, which takes blocks x, x + 8, ... (q or
  // q + 1 of them for ntiles = 8q + r); they get consecutive logical tiles from x q + min(x, r)
  const int xcd = blockIdx.x & 7, q8 = ntiles >> 3, r8 = ntiles & 7;
  const int pid = xcd * q8 + min(xcd, r8) + (blockIdx.x >> 3);
  const int group = pid / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (pid % (kGroupM * tiles_n)) % gsize;
  const int tn = (pid % (kGroupM * tiles_n)) / gsize;
  const int64_t m0 = static_cast<int64_t>(tm) * GBM, n0 = static_cast<int64_t>(tn) * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / WCOLS, wn = w % WCOLS;

  using AccV = typename std::conditional<F8, v16f, v16i>::type;   // fp32 or int32 accumulators
  using FragV = typename std::conditional<F8, v8i, v4i>::type;    // 32 or 16 K bytes per lane
  AccV acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int kbeg = 0;
  const int kend = g.k_dev ? min(static_cast<int>(g.K), max(0, *g.k_dev)) : static_cast<int>(g.K);
  const int KT = (kend - kbeg + GBK - 1) / GBK;
  // Operands go straight from memory into LDS (buffer loads with the lds bit): each wave
  // instruction fills 1 KB of LDS, lane l writing bytes 16l..16l+15, i.e. 16 rows of 64 bytes.
  // A lane fetches the global 16-byte chunk that the XOR swizzle of its LDS slot calls for.
  // Descriptors are rebased at the tile's first row: offsets past the valid rows (or the
  // sentinel used past K) read as zero, so edge tiles need no branches.
  const int rows_a = static_cast<int>(min<int64_t>(GBM, g.M - m0));
  const int rows_b = static_cast<int>(min<int64_t>(BN, g.N - n0));
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(g.a + m0 * g.lda), 0, static_cast<int>(rows_a * g.lda), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(g.b + n0 * g.ldb), 0, static_cast<int>(rows_b * g.ldb), kBufferFlags);
  constexpr int ABLK = GBM / RPB / NW;   // 1 KB blocks of A per wave per stage
  constexpr int BBLK = BN / RPB / NW;
  constexpr int NDMA = ABLK + BBLK;      // direct-to-LDS loads per wave per stage
  int oa[ABLK], ob[BBLK], ka[ABLK], kb[BBLK];
  {
    const int rr = lane / KC, pc = lane % KC;
#pragma unroll
    for (int i = 0; i < ABLK; ++i) {
      const int row = RPB * (w + NW * i) + rr;
      // logical chunk whose swizzled slot is this lane's (lds_off(row, lc) == block + 16 lane)
      const int lc = pc ^ ((lds_off<GBK>(row, 0) >> 4) & (KC - 1));
      oa[i] = row * static_cast<int>(g.lda) + 16 * lc;
      ka[i] = 16 * lc;
    }
#pragma unroll
    for (int i = 0; i < BBLK; ++i) {
      const int row = RPB * (w + NW * i) + rr;
      const int lc = pc ^ ((lds_off<GBK>(row, 0) >> 4) & (KC - 1));
      ob[i] = row * static_cast<int>(g.ldb) + 16 * lc;
      kb[i] = 16 * lc;
    }
  }
  auto dma = [&](int kt, int8_t* stg) {
    const int k0 = kbeg + kt * GBK;
#pragma unroll
    for (int i = 0; i < ABLK; ++i)
      lds_dma16(rsa, stg + (w + NW * i) * 1024, (k0 + ka[i] < kend) ? oa[i] + k0 : kOutOfRange);
#pragma unroll
    for (int i = 0; i < BBLK; ++i)
      lds_dma16(rsb, stg + A_BYTES + (w + NW * i) * 1024, (k0 + kb[i] < kend) ? ob[i] + k0 : kOutOfRange);
  };
  // fragment registers. Slice ks of a 128-byte step: int8, lane half h reads chunk 2 ks + h
  // (16 bytes), in two sets (ping-pong between slices); FP8, chunks 4 ks + h and 4 ks + 2 + h
  // (32 bytes), the same two for A and B, in one set (two would not fit beside the 128
  // accumulators: the slice's MFMAs are issued before the next slice's reads).
  constexpr int NSET = F8 ? 1 : 2;
  FragV af[NSET][4], bf[NSET][NB];
  auto frag = [&](int set, const int8_t* sa, int ks) {
    const int8_t* sb = sa + A_BYTES;
    if constexpr (F8) {
      const int c0 = 4 * ks + (lane >> 5), c1 = c0 + 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        const v4i lo = *reinterpret_cast<const v4i*>(sa + lds_off<GBK>(row, c0));
        const v4i hi = *reinterpret_cast<const v4i*>(sa + lds_off<GBK>(row, c1));
        af[set][i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int row = wn * WN + j * 32 + (lane & 31);
        const v4i lo = *reinterpret_cast<const v4i*>(sb + lds_off<GBK>(row, c0));
        const v4i hi = *reinterpret_cast<const v4i*>(sb + lds_off<GBK>(row, c1));
        bf[set][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    } else {
      const int ch = 2 * ks + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[set][i] = *reinterpret_cast<const v4i*>(sa + lds_off<GBK>(wm * 128 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bf[set][j] = *reinterpret_cast<const v4i*>(sb + lds_off<GBK>(wn * WN + j * 32 + (lane & 31), ch));
    }
  };
  auto mfma = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (F8)   // format 0 for both operands: FP8 E4M3; no block scales
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[set][i], bf[set][j],
                                                                      acc[i][j], 0, 0, 0, 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[set][i], bf[set][j], acc[i][j], 0, 0, 0);
      }
  };

  // Pipeline, one barrier per K step. At the start of step k, stage k is complete and
  // visible, fragment set 0 holds its first K slice, and (three stages) the loads of step k+1
  // are in flight. Step k: start the loads of step k+NST-1 into the stage last read in step
  // k-1 (whose reads every wave finished before that step's barrier); alternate between
  // reading the next slice into one fragment set and MFMAs on the other; before the last
  // slice's MFMAs, wait for this wave's loads of step k+1 and its own reads of stage k, then
  // barrier (stage k+1 is now complete for every wave) and read step k+1's first slice.
  // Loads past K read zeros.
  static_assert(NST == 2 || NDMA == 6 || NDMA == 3, "three-stage waits cover 3 or 6 loads per stage");
  auto wait_next = [&]() {
    if constexpr (NST == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (NDMA == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  };
  auto step = [&](int k, int8_t* cur, int8_t* nxt, int8_t* far) {
    dma(k + NST - 1, NST == 2 ? nxt : far);
    if constexpr (F8) {
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
        mfma(0);
        __builtin_amdgcn_sched_barrier(0);
        frag(0, cur, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma(0);
      __builtin_amdgcn_sched_barrier(0);
      wait_next();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      frag(0, nxt, 0);
    } else {
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
        frag(ks & 1, cur, ks);
        __builtin_amdgcn_sched_barrier(0);
        mfma((ks - 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_next();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      frag(0, nxt, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfma((KS - 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto last = [&](const int8_t* cur) {
    if constexpr (F8) {
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
        mfma(0);
        frag(0, cur, ks);
      }
      mfma(0);
    } else {
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
        frag(ks & 1, cur, ks);
        mfma((ks - 1) & 1);
      }
      mfma((KS - 1) & 1);
    }
  };

  if (KT > 0) {
    dma(0, st0);
    if constexpr (NST == 3) dma(1, st1);
    wait_next();
    __builtin_amdgcn_s_barrier();
    frag(0, st0, 0);
    // unrolled over the stages so every stage is a static LDS object (the compiler then waits
    // only for the loads a read depends on); the trailing steps run with stage pointers picked
    // at run time, and the last step has no successor
    int kt = 0;
    if constexpr (NST == 3) {
      for (; kt + 3 < KT; kt += 3) {
        step(kt, st0, st1, st2);
        step(kt + 1, st1, st2, st0);
        step(kt + 2, st2, st0, st1);
      }
    } else {
      for (; kt + 2 < KT; kt += 2) {
        step(kt, st0, st1, st2);
        step(kt + 1, st1, st0, st2);
      }
    }
    auto stg = [&](int i) { return i == 0 ? st0 : (i == 1 ? st1 : st2); };
    for (; kt + 1 < KT; ++kt) step(kt, stg(kt % NST), stg((kt + 1) % NST), stg((kt + 2) % NST));
    last(stg(kt % NST));
  }
  // every direct-to-LDS load (including the zero-filled ones past K) has landed before the
  // epilogue reuses the stages
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  if constexpr (EPI == EPI_I32) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < g.M && col < g.N) {
            if constexpr (F8) static_cast<float*>(g.c)[row * g.ldc + col] = acc[i][j][r];
            else static_cast<int32_t*>(g.c)[row * g.ldc + col] = acc[i][j][r];
          }
        }
      }
    return;
  } else {
    const float alpha = (*g.sa * *g.sb) * g.kmul;
    // (1) int32 -> fp32 in place, then the row (M) stages inside the accumulator layout
    v16f fa[4][NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (F8) fa[i][j] = acc[i][j];
        else fa[i][j] = __builtin_convertvector(acc[i][j], v16f);
      }
    if constexpr (KM > 1) {
      rows_fwht_inlane<KM, NB>(fa);
      // the row-major rounds apply the lane-half stage to each row block as they reach it
      if constexpr (KM > 4 && TRANS) rows_fwht_lanehalf<NB>(fa, lane);
    }
    // (2) two rounds through LDS, each holding 64 rows of both wave rows: rows 64 cc + [0, 64)
    // of wave row 0 in stage 0, the same rows of wave row 1 (tile rows + 128) in stage 1.
    // After the round's barrier a lane reads eight consecutive values of one output row from
    // each stage, so the row stride 128 is an in-register butterfly, and eight neighbouring
    // lanes cover 64 consecutive outputs: each 16-byte store instruction writes whole 128-byte
    // lines.
    float* const ep0 = reinterpret_cast<float*>(st0);
    float* const ep1 = reinterpret_cast<float*>(st1);
    float* const epw = wm ? ep1 : ep0;
    const int hh = lane >> 5, lq = lane & 31;
    const int s8 = lane & 7;
    auto bit7 = [&](float (&u0)[8], float (&u1)[8]) {
      if constexpr (KM > 128) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float a = u0[q], b = u1[q];
          u0[q] = a + b;
          u1[q] = a - b;
        }
      }
    };
    if constexpr (TRANS) {
      // Column-major rounds: element (row p < 64, column n) at n*64 + 4*((p/4) ^ (n%16)) + p%4:
      // a lane's four consecutive rows of the accumulator layout go in as one 16-byte write,
      // and both the writes and the reads below meet distinct bank groups. Lane (column n,
      // s8) then takes rows 8 s8 + [0, 8) of column n: eight elements of output row n0 + n.
      constexpr int PASSES = BN / 64;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        __syncthreads();
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int col = wn * WN + j * 32 + lq;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int gq = 8 * ib + 2 * rq + hh;
              const float4 x = {fa[2 * cc + ib][j][4 * rq], fa[2 * cc + ib][j][4 * rq + 1],
                                fa[2 * cc + ib][j][4 * rq + 2], fa[2 * cc + ib][j][4 * rq + 3]};
              *reinterpret_cast<float4*>(&epw[col * 64 + 4 * (gq ^ (col & 15))]) = x;
            }
          }
        __syncthreads();
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
          const int n = 64 * ps + 8 * w + (lane >> 3);
          float u0[8], u1[8];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int off = n * 64 + 4 * ((2 * s8 + k) ^ (n & 15));
            const float4 a = *reinterpret_cast<const float4*>(&ep0[off]);
            const float4 b = *reinterpret_cast<const float4*>(&ep1[off]);
            u0[4 * k] = a.x; u0[4 * k + 1] = a.y; u0[4 * k + 2] = a.z; u0[4 * k + 3] = a.w;
            u1[4 * k] = b.x; u1[4 * k + 1] = b.y; u1[4 * k + 2] = b.z; u1[4 * k + 3] = b.w;
          }
          bit7(u0, u1);
          const int64_t orow = n0 + n;
          const int64_t c0 = m0 + 64 * cc + 8 * s8, c1 = c0 + 128;
          if (orow < g.N) {
            if (g.nt) {
              store_run<Out, 8, false, true>(g.c, orow * g.ldc + c0, g.M - c0, u0, alpha);
              store_run<Out, 8, false, true>(g.c, orow * g.ldc + c1, g.M - c1, u1, alpha);
            } else {
              store_run<Out, 8>(g.c, orow * g.ldc + c0, g.M - c0, u0, alpha);
              store_run<Out, 8>(g.c, orow * g.ldc + c1, g.M - c1, u1, alpha);
            }
          }
        }
      }
    } else {
      // Four row-major rounds, one 32-row block of each wave row per round, rows padded to
      // BN + 4 floats (the 16-byte reads of two neighbouring rows by sixteen lanes meet
      // distinct bank groups, and every address is a lane base plus an immediate). Lane (row
      // x, s8) of wave half hh takes columns 64 jj + 8 s8 + [0, 8) of tile row
      // 32 cc + x + 128 hh: lanes l and l + 32 hold rows 128 apart (row stride 128 = one
      // v_permlane32_swap per value); column strides 1, 2, 4 and 64, 128 are in-register
      // butterflies, 8, 16 and 32 cross the eight lanes of a row (quad DPP, then a
      // bank-masked row shift).
      constexpr int NJ = BN / 64;
      constexpr int RP = BN + 4;           // padded row pitch (floats)
      const int x = 4 * w + (lq >> 3);
      const float* const epr = hh ? ep1 : ep0;
      // (store_rows: dn shifts the columns, for the pair finisher's lower / upper halves)
      // column strides 8 and 16 leave lane l's values multiplied by csgn (lane bits 0 and 1);
      // the sign goes into the scale of the stores, which negates them back exactly (a zero
      // is stored as +0, as the unfolded butterflies gave it)
      const float sg1 = (lane & 1) ? -1.0f : 1.0f, sg2 = (lane & 2) ? -1.0f : 1.0f;
      const float csgn = (KN > 8 ? sg1 : 1.0f) * (KN > 16 ? sg2 : 1.0f);
      const float alpha_l = alpha * csgn;
      auto store_rows = [&](int cc, const float (&u)[NJ][8], int dn) {
        const int64_t orow = m0 + 128 * hh + 32 * cc + x;
        if (orow < g.M) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) {
            const int64_t cb = n0 + dn + 64 * jj + 8 * s8;
            if (g.nt) store_run<Out, 8, true, true>(g.c, orow * g.ldc + cb, g.N - cb, u[jj], alpha_l);
            else store_run<Out, 8, true>(g.c, orow * g.ldc + cb, g.N - cb, u[jj], alpha_l);
          }
        }
      };
      // STASH: with the two-sided 128- and 256-point rotations, all 128 values of a lane plus a
      // round's working set do not fit the 256 registers a wave has at two waves per SIMD, and
      // the compiler would spill about 31 values to scratch memory (written and read back
      // through the caches for every tile). Instead the last round's block fa[3] (32 values)
      // goes to LDS once the row stages that mix the blocks are done and comes back when its
      // round starts: eight 16-byte chunks per thread, three past a round's 32 padded rows in
      // stage 0, three in stage 1, two in stash_x. Each thread reads only what it wrote, and
      // the rounds never touch these bytes, so no barrier is involved.
      constexpr int EP_ROUND = 32 * RP * 4;   // bytes of one round in a stage
      static_assert(!STASH || (EP_ROUND % 16 == 0 && EP_ROUND + 3 * NT * 16 <= STAGE),
                    "three stash chunks must fit past a round in each stage");
      auto stash_at = [&](int c) -> float4* {
        if (c < 3) return reinterpret_cast<float4*>(st0 + EP_ROUND + c * NT * 16) + t;
        if (c < 6) return reinterpret_cast<float4*>(st1 + EP_ROUND + (c - 3) * NT * 16) + t;
        return &stash_x[(c - 6) * NT + t];
      };
      if constexpr (STASH) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int j = c / 4, e = 4 * (c % 4);
          *stash_at(c) = make_float4(fa[3][j][e], fa[3][j][e + 1], fa[3][j][e + 2], fa[3][j][e + 3]);
        }
      }
      float res[PAIR ? 4 : 1][NJ][8];   // PAIR: this tile's rotated values, kept for the exchange
      // PAIR: the tile's column half, and its published values (device-coherent sc1 stores)
      const int half = tn & 1;
      constexpr int SLOT = NT * 4 * NJ * 8 * 4;    // bytes of one published tile
      constexpr int kDeviceScope = 16;              // cache policy: sc1
      const int64_t pair_id = static_cast<int64_t>(tm) * (tiles_n >> 1) + (tn >> 1);
      auto pair_rsrc = [&]() {
        return __builtin_amdgcn_make_buffer_rsrc(g.pair_part + pair_id * 2 * (SLOT / 4), 0, 2 * SLOT,
                                                 kBufferFlags);
      };
      auto slot = [&](int part, int cc, int jj, int k) {
        return part * SLOT + (((cc * NJ + jj) * 2 + k) * NT + t) * 16;
      };
      auto publish = [&](const __amdgpu_buffer_rsrc_t& rsp, int cc) {
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float4 f = {res[cc][jj][4 * k], res[cc][jj][4 * k + 1], res[cc][jj][4 * k + 2],
                              res[cc][jj][4 * k + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, f), rsp, slot(half, cc, jj, k),
                                                   0, kDeviceScope);
          }
      };
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        if constexpr (STASH) {
          if (cc == 3) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const float4 v = *stash_at(c);
              const int j = c / 4, e = 4 * (c % 4);
              fa[3][j][e] = v.x; fa[3][j][e + 1] = v.y; fa[3][j][e + 2] = v.z; fa[3][j][e + 3] = v.w;
            }
          }
        }
        if constexpr (KM > 4) rows_fwht_lanehalf_block<NB>(fa[cc], lane);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = wn * WN + j * 32 + lq;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pr = 8 * (r >> 2) + 4 * hh + (r & 3);
            epw[pr * RP + col] = fa[cc][j][r];
          }
        }
        __syncthreads();
        float u[NJ][8];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float4 a = *reinterpret_cast<const float4*>(&epr[x * RP + 64 * jj + 8 * s8 + 4 * k]);
            u[jj][4 * k] = a.x; u[jj][4 * k + 1] = a.y; u[jj][4 * k + 2] = a.z; u[jj][4 * k + 3] = a.w;
          }
        float* const f = &u[0][0];
        if constexpr (KM > 128) {
          // row stride 128 = lane bit 5, two values per pair of swaps as in the row stages
#pragma unroll
          for (int q = 0; q < 8 * NJ; q += 2) {
            auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(f[q]), __float_as_uint(f[q + 1]),
                                                       false, false);
            const float lo = __uint_as_float(pr[0]), hi = __uint_as_float(pr[1]);
            auto qr = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo + hi),
                                                       __float_as_uint(lo - hi), false, false);
            f[q] = __uint_as_float(qr[0]);
            f[q + 1] = __uint_as_float(qr[1]);
          }
        }
        if constexpr (KN > 1) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) fwht_inreg<KN, 8>(u[jj]);
          // strides 8, 16 = lane bits 0, 1: one fused DPP fma per value, the upper lanes left
          // holding the negated butterfly output (csgn, folded into the store's scale)
          if constexpr (KN > 8) {
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
              xstage8<1>(u[jj][0], u[jj][1], u[jj][2], u[jj][3], u[jj][4], u[jj][5], u[jj][6],
                         u[jj][7], sg1);
          }
          if constexpr (KN > 16) {
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
              xstage8<2>(u[jj][0], u[jj][1], u[jj][2], u[jj][3], u[jj][4], u[jj][5], u[jj][6],
                         u[jj][7], sg2);
          }
          // stride 32 = lane bit 2: the partner is lane ^ 4 (two bank-masked row shifts); the
          // lanes of a pair carry the same csgn, so the stage needs no sign of its own
          if constexpr (KN > 32) {
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) xstage4_lane4(u[jj]);
          }
#pragma unroll
          for (int hb = 1; hb < NJ; hb <<= 1)
            if (64 * hb < KN) {
#pragma unroll
              for (int jj = 0; jj < NJ; ++jj)
                if ((jj & hb) == 0)
#pragma unroll
                  for (int q = 0; q < 8; ++q) {
                    const float a = u[jj][q], b = u[jj + hb][q];
                    u[jj][q] = a + b;
                    u[jj + hb][q] = a - b;
                  }
            }
        }
        if constexpr (PAIR) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int q = 0; q < 8; ++q) res[cc][jj][q] = u[jj][q];
          if (hh != half) publish(pair_rsrc(), cc);   // rows the partner finishes, sent at once
        } else {
          store_rows(cc, u, 0);
        }
      }
      if constexpr (PAIR) {
        // Column stride 128 of a 256-column rotation block spans the two 256 x 128 tiles of a
        // pair (tn even = lower column half). The tile of column half h finishes tile rows
        // 128h + [0, 128) of both column halves (its lanes with hh == h): lower half = sum of
        // the two tiles' values, upper half = lower-half tile's minus upper-half tile's. Each
        // tile published, during the rounds above, its values of the rows its partner finishes.
        // Flag bits: P_h (tile h published those rows), F_h (tile h published all rows and
        // left). A tile sets P, then waits a bounded time (pair_spin polls, ~0.5 us each) for
        // the partner's P; normally both see both bits and each finishes its own rows. After
        // the bound (the partner may not be running yet) it publishes its remaining rows, sets
        // F and leaves, unless the partner's P appeared meanwhile; a tile that finds the
        // partner's F set finishes all rows. No tile waits without bound, and every output is
        // written (twice, with equal values, in the narrow race where both finish all). Values
        // move with device-coherent (sc1) buffer stores and loads: the stores are complete
        // (s_waitcnt) before the flag's atomic and the loads issue after the partner's bit is
        // seen, so no cache-wide writeback or invalidate is needed. The flags start at zero
        // (cleared by the launch before on the stream) and are left set: a tile still polling
        // must not see its partner's bit disappear.
        __shared__ int s_state;
        const __amdgpu_buffer_rsrc_t rsp = pair_rsrc();
        const int pme = 1 << half, pother = 1 << (half ^ 1), fme = 4 << half, fother = 4 << (half ^ 1);
        int* flag = &g.pair_cnt[pair_id];
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t == 0) {
          int st = __hip_atomic_fetch_or(flag, pme, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int i = 0; i < g.pair_spin && !(st & pother); ++i) {
            __builtin_amdgcn_s_sleep(16);
            st = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          s_state = st;
        }
        __syncthreads();
        int st = s_state;
        if (!(st & pother)) {
          if (hh == half) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) publish(rsp, cc);
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (t == 0) s_state = __hip_atomic_fetch_or(flag, fme, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __syncthreads();
          st = s_state;
          if (!(st & pother)) return;
        }
        if (hh == half || (st & fother)) {
          const float sgn_own = half ? -1.0f : 1.0f;
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            float lo[NJ][8], up[NJ][8];
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
              for (int k = 0; k < 2; ++k) {
                const float4 f = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                    rsp, slot(half ^ 1, cc, jj, k), 0, kDeviceScope));
                const float pv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float own = res[cc][jj][4 * k + e];
                  lo[jj][4 * k + e] = own + pv[e];
                  up[jj][4 * k + e] = __builtin_fmaf(own, sgn_own, -sgn_own * pv[e]);
                }
              }
            store_rows(cc, lo, -BN * half);
            store_rows(cc, up, BN * (1 - half));
          }
        }
      }
    }
  }
}

template <int BN, class Out, int EPI, int KM, int KN, bool TRANS, bool PAIR, bool F8>
static hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int tok, int batch) {
  const int64_t tiles = ((a.M + GBM - 1) / GBM) * ((a.N + BN - 1) / BN);
  return launch_k(gemm_i8_kernel<BN, Out, EPI, KM, KN, TRANS, PAIR, F8>,
                  dim3(static_cast<int>(tiles), batch), dim3(GemmShape<BN>::NT), st, tok, a);
}

template <int BN, class Out, bool F8>
static hipError_t launch_out(const GemmPass& p, const GemmArgs& a, hipStream_t st, int tok) {
  if (p.trans_out) {
    switch (p.km) {
#define HQ_T(KK) case KK: return launch_gemm<BN, Out, EPI_SCALE, KK, 1, true, false, F8>(a, st, tok, p.batch);
      HQ_T(1) HQ_T(2) HQ_T(4) HQ_T(8) HQ_T(16) HQ_T(32) HQ_T(64) HQ_T(128) HQ_T(256)
#undef HQ_T
    }
    return hipErrorInvalidValue;
  }
  if (p.km == 1 && p.kn == 1) return launch_gemm<BN, Out, EPI_SCALE, 1, 1, false, false, F8>(a, st, tok, p.batch);
  if (p.km != p.kn) return hipErrorInvalidValue;
  if constexpr (BN == 128) {
    // column blocks up to 128 wide rotate inside the tile; 256-wide ones span a tile pair
    switch (p.km) {
#define HQ_B(KK) case KK: return launch_gemm<BN, Out, EPI_SCALE, KK, KK, false, false, F8>(a, st, tok, p.batch);
      HQ_B(2) HQ_B(4) HQ_B(8) HQ_B(16) HQ_B(32) HQ_B(64) HQ_B(128)
#undef HQ_B
      case 256:
        if (!a.pair_part) return hipErrorInvalidValue;
        return launch_gemm<BN, Out, EPI_SCALE, 256, 256, false, true, F8>(a, st, tok, p.batch);
    }
  } else {
    switch (p.km) {
#define HQ_B(KK) case KK: return launch_gemm<BN, Out, EPI_SCALE, KK, KK, false, false, F8>(a, st, tok, p.batch);
      HQ_B(2) HQ_B(4) HQ_B(8) HQ_B(16) HQ_B(32) HQ_B(64) HQ_B(128) HQ_B(256)
#undef HQ_B
    }
  }
  return hipErrorInvalidValue;
}

// 128-wide tiles when 256-wide ones would leave most CUs idle and every rotation fits: rows
// always (a tile holds 256 rows), columns when the block is at most 128 wide or, for 256, by
// pairing the two tiles of a block (N is then a multiple of 256: the rotated axis is a whole
// number of blocks).
static bool use_narrow(int64_t M, int64_t N, int kn, bool trans_out) {
  const int64_t tiles256 = ((M + GBM - 1) / GBM) * ((N + 255) / 256);
  if (tiles256 >= 256) return false;
  return kn <= 128 || (kn == 256 && !trans_out && N % 256 == 0);
}

// 256-wide tile columns to run before a second launch of 128-wide tiles over the rest of N,
// or tn for one launch. When the 256-wide grid leaves its last round of workgroups partly
// filled, a tail of 128-wide tiles can fill whole rounds instead. Estimated cost in rounds of
// 256 x 256 tiles: a full round 1, a round filled to a fraction f about 0.6 + 0.4 f (fewer
// workgroups share the memory system), a round of 256 x 128 tiles 0.6 of that (measured
// K-loop rates 2.6 and 3.1 POP/s), the extra launch 0.05. The tail needs no tile pairs.
static int64_t wide_cols_before_tail(int64_t tm, int64_t tn, int cus) {
  auto rounds = [cus](int64_t tiles) {
    const int64_t full = tiles / cus, rem = tiles % cus;
    return static_cast<double>(full) + (rem ? 0.6 + 0.4 * static_cast<double>(rem) / cus : 0.0);
  };
  double best = rounds(tm * tn);
  int64_t best_n1 = tn;
  for (int64_t n1 = 1; n1 < tn; ++n1) {
    const double c = rounds(tm * n1) + 0.6 * rounds(tm * 2 * (tn - n1)) + 0.05;
    if (c < best - 1e-9) {
      best = c;
      best_n1 = n1;
    }
  }
  return best_n1;
}

int64_t gemm_split_tiles(int64_t M, int64_t N, int64_t K, int epi, int km, int kn, bool trans_out) {
  (void)K;
  (void)km;
  if (epi != EPI_SCALE || kn != 256 || !use_narrow(M, N, kn, trans_out)) return 0;
  return ((M + GBM - 1) / GBM) * (N / 256);   // tile pairs
}

size_t gemm_split_bytes(int64_t pairs) {
  // arrival flags (rounded to 256 B), then two published tiles of 512 threads x 64 fp32 per pair
  return static_cast<size_t>((pairs * 4 + 255) / 256 * 256) +
         static_cast<size_t>(pairs) * 2 * 512 * 64 * 4;
}

hipError_t gemm_pass(const GemmPass& p, hipStream_t st) {
  GemmArgs a{p.a, p.lda, p.b, p.ldb, p.M, p.N, p.K, p.c, p.ldc, p.sa, p.sb, p.kmul,
             nullptr, nullptr, 40, p.a_bstride, p.b_bstride, p.c_bstride, p.k_dev};
  if (p.batch < 1 || p.batch > 65535) return hipErrorInvalidValue;
  // Test hook: HQ_PAIR_SPIN bounds the tile-pair wait (40 polls of ~0.5 us by default); 0 makes
  // every early tile take the wait-free fallback, which tests use to cover that path.
  if (const char* e = std::getenv("HQ_PAIR_SPIN")) a.pair_spin = std::max(0, std::atoi(e));
  // The outputs leave with the non-temporal hint: nothing later in the call reads them, and
  // kept in the caches they only displace operands and leave dirty lines for the next
  // memory-bound pass to write back. At 8192 x 13824 x 5120 the step went 1.891 -> 1.870 ms
  // (GEMMs 1.537 -> 1.500 ms, the absmax passes 132 -> 116 us), at 4096 x 4096 x 11008
  // 0.737 -> 0.704 ms. HQ_GEMM_NT=0 stores them normally.
  a.nt = 1;
  if (const char* e = std::getenv("HQ_GEMM_NT")) a.nt = (e[0] == '0') ? 0 : 1;
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const int64_t pairs =
      p.batch > 1 ? 0 : gemm_split_tiles(p.M, p.N, p.K, p.epi, p.km, p.kn, p.trans_out);
  if (pairs > 0) {
    if (!p.split_ws) return hipErrorInvalidValue;
    a.pair_cnt = static_cast<int32_t*>(p.split_ws);
    a.pair_part = reinterpret_cast<float*>(static_cast<char*>(p.split_ws) + (pairs * 4 + 255) / 256 * 256);
    if (!p.split_cnt_zeroed) {
      const hipError_t e = zero_i32(a.pair_cnt, pairs, st);
      if (e != hipSuccess) return e;
    }
  }
  // a tile's rows must be addressable by 32-bit buffer offsets
  if (static_cast<int64_t>(GBM) * p.lda >= kOutOfRange || 256 * p.ldb >= kOutOfRange)
    return hipErrorInvalidValue;
  const int kn = p.epi == EPI_I32 ? 1 : p.kn;
  // batched: every batch's tiles count towards filling the device; 256-wide column blocks
  // stay inside one tile (no tile pairs across a batch), and there is no tail launch
  const bool narrow = p.batch > 1
                          ? (((p.M + GBM - 1) / GBM) * ((p.N + 255) / 256) * p.batch < 256 && kn <= 128)
                          : use_narrow(p.M, p.N, kn, p.trans_out);
  auto launch_fmt = [&](bool nar, const GemmArgs& g, auto f8) -> hipError_t {
    constexpr bool F8 = decltype(f8)::value;
    const int tok = prof_open(K_GEMM, 2.0 * g.M * g.N * g.K * p.batch);
    if (p.epi == EPI_I32)
      return nar ? launch_gemm<128, F32, EPI_I32, 1, 1, false, false, F8>(g, st, tok, p.batch)
                 : launch_gemm<256, F32, EPI_I32, 1, 1, false, false, F8>(g, st, tok, p.batch);
    switch (p.out_dt) {
      case DT_F32: return nar ? launch_out<128, F32, F8>(p, g, st, tok) : launch_out<256, F32, F8>(p, g, st, tok);
      case DT_F16: return nar ? launch_out<128, F16, F8>(p, g, st, tok) : launch_out<256, F16, F8>(p, g, st, tok);
      case DT_BF16: return nar ? launch_out<128, BF16, F8>(p, g, st, tok) : launch_out<256, BF16, F8>(p, g, st, tok);
    }
    return hipErrorInvalidValue;
  };
  auto launch = [&](bool nar, const GemmArgs& g) {
    return p.f8 ? launch_fmt(nar, g, std::true_type{}) : launch_fmt(nar, g, std::false_type{});
  };
  if (!narrow && kn <= 128 && p.batch == 1) {
    // 256-wide tiles over columns [0, N1), then 128-wide ones over [N1, N) when that fills the
    // rounds better (N1 is a multiple of 256, so rotation blocks stay whole in each part)
    const int64_t tm = (p.M + GBM - 1) / GBM, tn = (p.N + 255) / 256;
    const int64_t n1 = wide_cols_before_tail(tm, tn, p.cus > 0 ? p.cus : 256) * 256;
    if (n1 < p.N) {
      const size_t esz = p.epi == EPI_I32 ? 4 : (p.out_dt == DT_F32 ? 4 : 2);
      GemmArgs head = a, tail = a;
      head.N = n1;
      tail.N = p.N - n1;
      tail.b = p.b + n1 * p.ldb;
      // c is M x N (pitch ldc), or N x M when the transpose is stored
      tail.c = static_cast<char*>(p.c) + static_cast<size_t>(p.trans_out ? n1 * p.ldc : n1) * esz;
      const hipError_t e = launch(false, head);
      if (e != hipSuccess) return e;
      return launch(true, tail);
    }
  }
  return launch(narrow, a);
}

}  // namespace hq
