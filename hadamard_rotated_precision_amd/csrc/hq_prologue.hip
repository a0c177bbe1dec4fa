// hq_prologue.hip — the rotate -> tensor-wise scale -> quantize prologue of HQ-MM for gfx950.
//
// "Training Transformers with 4-bit Integers", §3.3 (block-diagonal H_k transform before
// quantization), §3.1 (symmetric integer grid, learned step), §A.6 (Hadamard multiplication,
// quantization and packing before the integer GEMM; the GEMM wants K-contiguous operands, so
// the transposed codes a backward product reads are written here rather than by a separate
// transpose); "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs", Approach (right
// rotation of X and W, left rotation of dY, one scale per tensor).
//
// Each kernel runs twice per tensor: an absmax pass (one partial max per workgroup, reduced by
// the next pass, so no atomics and an order-independent result) and a quantize pass that
// recomputes the rotation and writes codes. In STEP mode only the quantize pass runs.
//
// Matrix-core kernels (16-bit inputs of whole tiles, k >= 16): the rotation is the product with
// blockdiag(H_k) on v_mfma_f32_16x16x32_{bf16,f16} in blocks of up to 64, plus in-register
// butterflies for the strides 64 and 128.
//   right_mma_kernel : along the contiguous axis (W; X under HQ), 64 x 256 tiles.
//   left_mma_kernel  : along the token axis (dY under HALO-2), 256 x 64 tiles staged raw in LDS,
//                      H fragments as the A operand.
//   both_mma_kernel  : X under HALO-2, 256 x 256 tiles: the row phase on the matrix cores, the
//                      half tile staged column-major, the token phase in TokenT (fp32);
//                      both_pipe_kernel is the same with the next item's raw rows loaded into
//                      LDS during the current item's token phase (several items per workgroup).
//   both_narrow_kernel : the same for k <= 128 on 128 x 128 items: 64 KB of LDS per workgroup of
//                      four waves, two workgroups per CU (the default where both_pipe_kernel
//                      would run and k <= 128).
// VALU kernels (every other shape: fp32 inputs, k < 16, ragged tiles, unaligned pitches):
//   right_fast_kernel / right_kernel : rotation along the contiguous axis. Tile 64 rows x 256
//                  columns; four lanes share a row, so strides < 64 are in-register butterflies
//                  and the rest DPP exchanges. Transposed codes go through LDS.
//   left_fast_kernel / left_kernel : rotation along rows (the token axis). The tile is staged in
//                  LDS as fp32 with a column swizzle; a thread then owns 64 consecutive rows of
//                  one column (in-register butterflies) and four lanes share a column.
//   both_kernel  : X under HALO-2, 256 x 256 tiles, 512 threads: the right rotation (two rows
//                  per thread) feeds the row-major codes of Q(X B); the same registers, staged
//                  through LDS in two 128-column halves, feed the token-axis rotation (64 rows of
//                  one column per thread) whose codes Q(B X B) are written transposed.
#include <algorithm>
#include <cstdlib>

#include "hq_device.hpp"
#include "hq_internal.hpp"
#include "hq_launch.hpp"

namespace hq {

// 64 consecutive elements starting at element c0 of a row with n valid elements.
template <class T>
__device__ inline void load64(const void* row, int64_t c0, int64_t n, bool vec, float (&v)[64]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float u[16];
    load16<T>(row, c0 + 16 * q, n, vec && (c0 + 16 * q + 16 <= n), u);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[16 * q + j] = u[j];
  }
}

// Pack 16 codes starting at v[i0] into a uint4 (integer codes, or E4M3 codes when f8).
__device__ inline uint4 pack16(const float (&v)[64], int i0, float r, int qp, bool f8, float grid,
                              float fmax) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = f8 ? fcode_pack4(v[i0 + 4 * j], v[i0 + 4 * j + 1], v[i0 + 4 * j + 2], v[i0 + 4 * j + 3], r,
                            grid, fmax)
              : pack4(quant_code(v[i0 + 4 * j], r, qp), quant_code(v[i0 + 4 * j + 1], r, qp),
                      quant_code(v[i0 + 4 * j + 2], r, qp), quant_code(v[i0 + 4 * j + 3], r, qp));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

struct ProArgs {
  const void* src;
  int64_t rows, cols;
  bool vec;                 // 16-byte loads allowed (row pitch and base aligned)
  float* partials;          // ABSMAX out (both_kernel: [0, grid) right, [grid, 2*grid) both)
  const float* part_in;     // QUANT in
  const float* part_in2;    // both_kernel QUANT: partials of the two-sided rotation
  int nparts;
  const float* step;        // QUANT, STEP mode (right / left rotation, or X B for both_kernel)
  const float* step2;       // both_kernel, STEP mode: step of B X B
  int qp;                   // integer codes: the grid bound 127 / 7
  float qmaxf;              // the scale's divisor: Qp, or the float format's largest value
  int fgrid;                // float-format codes: 0 E4M3, 1 E2M3, 2 E3M2 (FP6, as E4M3 bytes)
  float* scale_out;
  float* scale_out2;        // both_kernel: scale of B X B
  int8_t* codes;            // row-major codes (pitch ld) or nullptr
  int64_t ld;
  int8_t* codes_t;          // transposed codes (pitch ld_t) or nullptr
  int64_t ld_t;
  int32_t* zero_ptr;        // QUANT: block 0 zeroes these ints for a later launch
  int64_t zero_n;
  int32_t* bar;             // both_single_kernel: barrier words (zeroed by the launch before);
                            // a QUANT pass given bar runs only if the single pass aborted
  int spin;                 // both_single_kernel: polls of the barrier before giving up
  void* dst;                // right/left_mma_kernel OP_STORE: rotated values, rows x cols, input dtype
  int rev;                  // right/left_mma, both_narrow QUANT: visit the tiles last to first
};

// Barrier words of the single-pass two-sided kernel: arrival counters of eight workgroup groups
// (128 bytes apart), the group-completion counter and the state word (0 open, 1 released,
// 2 aborted).
constexpr int kBarGroups = 8, kBarStride = 32, kGroupDone = 256, kReleaseWord = 288,
              kStateAborted = 2;

// A quantize pass (integer or FP8 codes).
__host__ __device__ constexpr bool quant_op(int op) { return op == OP_QUANT || op == OP_QUANT_F8; }

// The (lo, hi) pair quant4 takes: the integer clamp bounds, or for float-format codes the grid
// and the format's largest value.
template <int OP>
__device__ inline float code_lo(const ProArgs& a) {
  return OP == OP_QUANT_F8 ? static_cast<float>(a.fgrid) : qlo(a.qp);
}
template <int OP>
__device__ inline float code_hi(const ProArgs& a) {
  return OP == OP_QUANT_F8 ? a.qmaxf : qhi(a.qp);
}

// Counters a later launch on the stream needs at zero (the split-K arrivals of the GEMM).
__device__ inline void zero_side(const ProArgs& a) {
  if (a.zero_n > 0 && blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < a.zero_n; i += blockDim.x) a.zero_ptr[i] = 0;
}

// ================================================================ right rotation
constexpr int RT_ROWS = 64, RT_COLS = 256, RT_THREADS = 256;

template <class In, int K, int OP>
__global__ __launch_bounds__(RT_THREADS) void right_kernel(ProArgs a) {
  __shared__ float red[32];
  __shared__ __attribute__((aligned(16))) int8_t tcodes[RT_COLS][RT_ROWS + 16];
  const int t = threadIdx.x, lane = t & 63;
  const int r = t >> 2, s = t & 3;   // tile row, 64-column segment
  const int64_t nrt = (a.rows + RT_ROWS - 1) / RT_ROWS, nct = (a.cols + RT_COLS - 1) / RT_COLS;
  const int64_t tiles = nrt * nct;
  float sc = 0.0f, rinv = 0.0f;
  if constexpr (quant_op(OP)) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, sc, rinv);
    zero_side(a);
    if (blockIdx.x == 0 && t == 0) *a.scale_out = sc;
  }
  const int64_t rpad = (a.rows + 15) / 16 * 16;   // valid extent of a transposed row
  float amax = 0.0f;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t row0 = (tile / nct) * RT_ROWS, col0 = (tile % nct) * RT_COLS;
    const int64_t grow = row0 + r, gc = col0 + 64 * s;
    float v[64];
    if (grow < a.rows && gc < a.cols) {
      load64<In>(static_cast<const char*>(a.src) + grow * a.cols * In::bytes, gc, a.cols, a.vec, v);
    } else {
#pragma unroll
      for (int j = 0; j < 64; ++j) v[j] = 0.0f;
    }
    fwht_inreg<K, 64>(v);
    if constexpr (K > 64) quad_stage<64>(v, lane, 1);
    if constexpr (K > 128) quad_stage<64>(v, lane, 2);
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(v[j]));
    } else {
      // row-major codes: 64 consecutive bytes, written up to the 16-byte-padded row end
      if (a.codes && grow < a.rows) {
        int8_t* dst = a.codes + grow * a.ld + gc;
        const int64_t cpad = (a.cols + 15) / 16 * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (gc + 16 * q < cpad) *reinterpret_cast<uint4*>(dst + 16 * q) = pack16(v, 16 * q, rinv, a.qp, (OP == OP_QUANT_F8), static_cast<float>(a.fgrid), a.qmaxf);
      }
      if (a.codes_t) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 64; ++j)
          tcodes[64 * s + j][r] = static_cast<int8_t>(quant_byte(v[j], rinv, a.qp, (OP == OP_QUANT_F8), static_cast<float>(a.fgrid), a.qmaxf));
        __syncthreads();
        // thread t writes transposed row col0 + t: 64 bytes = tile rows row0 .. row0+63
        const int64_t orow = col0 + t;
        if (orow < a.cols) {
          int8_t* dst = a.codes_t + orow * a.ld_t + row0;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (row0 + 16 * q < rpad)
              *reinterpret_cast<uint4*>(dst + 16 * q) = *reinterpret_cast<const uint4*>(&tcodes[t][16 * q]);
        }
      }
    }
  }
  if constexpr (OP == OP_ABSMAX) {
    amax = block_max(amax, red);
    if (t == 0) a.partials[blockIdx.x] = amax;
  }
}

// ================================================================ right rotation, full tiles
// Used when the tensor is whole 64 x 256 tiles with 16-byte aligned rows. Persistent
// workgroups walk the tiles and load the next tile's row segment into registers before
// working on the current one, so memory and ALU overlap.
constexpr int RF_ROWS = 64, RF_COLS = 256, RF_THREADS = 256, RF_GRID = 512;

template <int M>
__device__ inline void xstage_signed(float (&v)[64], float sgn) {
#pragma unroll
  for (int i = 0; i < 64; i += 8)
    xstage8<M>(v[i], v[i + 1], v[i + 2], v[i + 3], v[i + 4], v[i + 5], v[i + 6], v[i + 7], sgn);
}

// 64 raw elements (4*bytes uint4) to fp32, with the stride-1 butterfly applied when K >= 2
// (v_dot2 on the packed pairs of 16-bit inputs).
template <class In, int K>
__device__ inline void unpack64(const uint4 (&c)[4 * In::bytes], float (&v)[64]) {
  if constexpr (In::bytes == 2) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t w[4] = {c[q].x, c[q].y, c[q].z, c[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* o = &v[8 * q + 2 * j];
        if constexpr (K >= 2) {
          if constexpr (In::is_bf16) {
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            const b2 x = __builtin_bit_cast(b2, w[j]);
            o[0] = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(b2, 0x3F803F80u), 0.0f, false);
            o[1] = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(b2, 0xBF803F80u), 0.0f, false);
          } else {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            const h2 x = __builtin_bit_cast(h2, w[j]);
            o[0] = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(h2, 0x3C003C00u), 0.0f, false);
            o[1] = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(h2, 0xBC003C00u), 0.0f, false);
          }
        } else {
          o[0] = In::from_bits(static_cast<uint16_t>(w[j] & 0xFFFFu));
          o[1] = In::from_bits(static_cast<uint16_t>(w[j] >> 16));
        }
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      v[4 * q] = __uint_as_float(c[q].x);
      v[4 * q + 1] = __uint_as_float(c[q].y);
      v[4 * q + 2] = __uint_as_float(c[q].z);
      v[4 * q + 3] = __uint_as_float(c[q].w);
    }
    if constexpr (K >= 2) fwht_inreg<2, 64>(v);
  }
}

__host__ __device__ inline bool right_fast_ok(int64_t rows, int64_t cols, bool vec) {
  return vec && rows > 0 && cols > 0 && rows % RF_ROWS == 0 && cols % RF_COLS == 0 &&
         (rows / RF_ROWS) * (cols / RF_COLS) < (int64_t(1) << 31);
}

// Tile 64 x 256. Thread (r = t/4, s = t%4) owns 64 elements of row r, interleaved so that
// each load instruction reads 64 contiguous bytes per row: its v[8j + i] is column
// 32j + 8s + i (j, i < 8). Butterfly strides 1, 2, 4 (column bits 0-2) and 32, 64, 128 (bits
// 5-7) are in-register; strides 8 and 16 (bits 3, 4 = lane bits 0, 1) are quad DPP stages.
// Transposed codes: the dwords of four codes along a row are transposed as 4x4 byte blocks
// across the four lanes that hold rows 4i..4i+3 (DPP row_ror:8, then row_shl/shr:4 with bank
// masks, each followed by a v_perm), which leaves each lane four consecutive rows of one
// column; these go to LDS as dwords (16-byte chunks XOR-swizzled so that both the dword
// writes and the 16-byte reads are conflict-free) and leave as 64-byte rows of the transpose.
__device__ inline int rf_swz(int c) { return ((c >> 2) & 3) ^ ((c >> 4) & 3); }

template <int K>
__device__ inline void right_stages(float (&v)[64], float sg1, float sg2) {
#pragma unroll
  for (int h = 2; h <= 4; h <<= 1) {       // column strides 2, 4 (stride 1 came with the load)
    if (h < K) {
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & h) == 0) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
    }
  }
  if constexpr (K > 8) xstage_signed<1>(v, sg1);    // column stride 8
  if constexpr (K > 16) xstage_signed<2>(v, sg2);   // column stride 16
#pragma unroll
  for (int h = 8; h <= 32; h <<= 1) {      // column strides 32, 64, 128
    if (4 * h < K) {
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & h) == 0) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
    }
  }
}

template <class In, int K, int OP>
__global__ __launch_bounds__(RF_THREADS) void right_fast_kernel(ProArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t tc[RF_COLS * 16];
  __shared__ float red[32];
  const int t = threadIdx.x, lane = t & 63;
  const int r = t >> 2, s = t & 3;
  const uint32_t nct = static_cast<uint32_t>(a.cols / RF_COLS);
  const uint32_t tiles = static_cast<uint32_t>(a.rows / RF_ROWS) * nct;   // < 2^31 (host checks)
  float sc = 0.0f, rinv = 0.0f;
  if constexpr (quant_op(OP)) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, sc, rinv);
    zero_side(a);
    if (blockIdx.x == 0 && t == 0) *a.scale_out = sc;
  }
  constexpr int XMASK = K > 16 ? 3 : (K > 8 ? 1 : 0);
  const float rr = (__builtin_popcount(lane & XMASK) & 1) ? -rinv : rinv;
  const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
  const float sg1 = (lane & 1) ? -1.0f : 1.0f, sg2 = (lane & 2) ? -1.0f : 1.0f;
  constexpr int NQ = 4 * In::bytes;      // 16-byte chunks per thread per tile
  constexpr int PER = 16 / In::bytes;    // elements per chunk
  const char* src = static_cast<const char*>(a.src);
  auto issue = [&](uint32_t tl, uint4 (&raw)[NQ]) {
    const uint32_t tr = tl / nct;
    const int64_t row = static_cast<int64_t>(tr) * RF_ROWS + r;
    const int64_t col = static_cast<int64_t>(tl - tr * nct) * RF_COLS + 8 * s;
    const char* p = src + (row * a.cols + col) * In::bytes;
#pragma unroll
    for (int q = 0; q < NQ; ++q)   // chunk q: columns 32*(q*PER/8) + 8s + (q*PER)%8 ...
      raw[q] = *reinterpret_cast<const uint4*>(p + (32 * ((q * PER) / 8) + (q * PER) % 8) * In::bytes);
  };
  uint4 rawA[NQ], rawB[NQ];
  uint32_t tl = blockIdx.x;
  if (tl < tiles) issue(tl, rawA);
  float amax = 0.0f;
  // one tile in registers while the next one loads: two register sets, alternating
  auto body = [&](const uint32_t tl, const uint4 (&cur)[NQ]) {
    float v[64];
    unpack64<In, K>(cur, v);
    right_stages<K>(v, sg1, sg2);
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(v[j]));
    } else {
      uint32_t d[16];   // d[g]: columns 32(g/2) + 8s + 4(g%2) + 0..3
#pragma unroll
      for (int g = 0; g < 16; ++g)
        d[g] = quant4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], rr, lo, hi, (OP == OP_QUANT_F8));
      const uint32_t tr = tl / nct;
      const int64_t row0 = static_cast<int64_t>(tr) * RF_ROWS;
      const int64_t col0 = static_cast<int64_t>(tl - tr * nct) * RF_COLS;
      if (a.codes) {
        int8_t* dst = a.codes + (row0 + r) * a.ld + col0 + 8 * s;
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint2*>(dst + 32 * j) = make_uint2(d[2 * j], d[2 * j + 1]);
      }
      if (a.codes_t) {
        const int b = (lane >> 2) & 3;                       // row within the 4-row block
        const uint32_t selA = (b < 2) ? 0x05040100u : 0x03020706u;
        const uint32_t selB = (b & 1) ? 0x03070105u : 0x06020400u;
        __syncthreads();   // the previous tile's readers of tc are done
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const uint32_t p = __builtin_amdgcn_mov_dpp(d[g], 0x128, 0xF, 0xF, false);   // lane ^ 8
          const uint32_t x = __builtin_amdgcn_perm(p, d[g], selA);
          uint32_t q = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0x5, false);           // lane + 4
          q = __builtin_amdgcn_update_dpp(q, x, 0x114, 0xF, 0xA, false);                     // lane - 4
          const uint32_t e = __builtin_amdgcn_perm(q, x, selB);
          const int c = 32 * (g >> 1) + 8 * s + 4 * (g & 1) + b;
          tc[c * 16 + ((r >> 2) ^ (4 * rf_swz(c)))] = e;
        }
        __syncthreads();
        const int x = rf_swz(t);
        uint4* dst = reinterpret_cast<uint4*>(a.codes_t + (col0 + t) * a.ld_t + row0);
        const uint4* sp = reinterpret_cast<const uint4*>(&tc[t * 16]);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = sp[j ^ x];
      }
    }
    };
  while (tl < tiles) {
    const uint32_t t1 = tl + gridDim.x;
    issue(t1 < tiles ? t1 : tl, rawB);   // unconditional: the last re-reads
    body(tl, rawA);
    if (t1 >= tiles) break;
    const uint32_t t2 = t1 + gridDim.x;
    issue(t2 < tiles ? t2 : t1, rawA);
    body(t1, rawB);
    tl = t2;
  }
  if constexpr (OP == OP_ABSMAX) {
    amax = block_max(amax, red);
    if (t == 0) a.partials[blockIdx.x] = amax;
  }
}

// ================================================================ right rotation on the matrix cores
// The row-axis rotation is the product X_tile . blockdiag(H_k): a dense contraction with +-1
// weights, run here on the 16-bit MFMA (v_mfma_f32_16x16x32_bf16 / _f16: exact products, fp32
// accumulation) so the VALU only quantizes and lays out codes. Used for 16-bit inputs, k >= 16,
// and tensors of whole 64 x 256 tiles with 16-byte aligned rows (right_fast_ok).
//
// Tile 64 x 256, four waves; wave w owns rows 16w .. 16w+15. K slice ks (32 columns) of the A
// operand: lane l holds row l%16, columns 32ks + 8(l/16) + [0, 8), so each load instruction reads
// 64 contiguous bytes per row. The B operand for output columns 16nb + [0, 16) is H_k restricted
// to that slice. With column c = 16c1 + c0, H_256 = H_16 (x) H_16 gives
// h(c, c') = h16(c1, c1') h16(c0, c0'); in a B fragment c0 and c0' depend on the lane and register
// only (lane l, element j: c0 = 8((l/16)%2) + j, c0' = l%16), and h16(c1, c1') with
// c1 = 2ks + l/32 splits into the compile-time sign h16(2ks, nb) times (-1)^((l/32) nb), so every
// fragment is one of four per-lane constants (G0, G1 = G0 with lanes 32..63 negated, and their
// negations). The matrix cores take blocks of at most 64 columns (c1, c1' modulo 4, slices
// outside the block skipped; k = 16 keeps only the lanes with l/32 = nb%2); for k = 128 and 256
// the column strides 64 and 128 are in-register butterflies between the nb blocks, which keeps
// the MFMA work at 32 instructions per wave and tile, below the VALU and memory time.
//
// Output of a 16 x 16 block: lane l holds rows 4(l/16) + [0, 4) of column 16nb + l%16, so four
// codes along a column pack into one dword of the transposed codes. Row-major codes come from a
// 4 x 4 byte transpose across the lanes of a quad (columns 4m + [0, 4), DPP quad_perm + v_perm).
// Both code tiles go through LDS as dwords, XOR-swizzled so that the dword writes and the 16-byte
// reads are conflict-free, and leave in 64-byte (transposed) and 256-byte (row-major) runs.
constexpr int RM_ROWS = 64, RM_COLS = 256, RM_THREADS = 256, RM_GRID = 512;

__host__ __device__ inline bool right_mma_ok(int64_t rows, int64_t cols, bool vec, int in_bytes,
                                             int k) {
  return in_bytes == 2 && k >= 16 && k <= RM_COLS && right_fast_ok(rows, cols, vec);
}

template <class In>
__device__ inline f32x4 mma16(const uint4& a, const uint4& b, const f32x4& c) {
  if constexpr (In::is_bf16) {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                    c, 0, 0, 0);
  } else {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                   c, 0, 0, 0);
  }
}

// B fragments of the +-1 contraction with blocks of KM <= 64 columns, G[2 * sign + nb % 2]:
// element j of lane l in G0 is h16(8((l/16)%2) + j, l%16); G1 negates lanes 32..63 (the factor
// (-1)^((l/32) nb) of h16(c1, c1')); G[2], G[3] are the negations. For KM = 16 the fragments
// keep only the lanes whose column block c1 = 2ks + l/32 is the output block nb.
template <class In, int KM>
__device__ inline void hfrags(int lane, uint4 (&G)[4]) {
  constexpr uint32_t ONE = In::is_bf16 ? 0x3F80u : 0x3C00u, SGN = 0x80008000u;
  const int n0 = lane & 15, lg = lane >> 4;
  uint32_t g0[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ca = 8 * (lg & 1) + 2 * i;
    const uint32_t e0 = ONE | ((__builtin_popcount(ca & n0) & 1) << 15);
    const uint32_t e1 = ONE | ((__builtin_popcount((ca + 1) & n0) & 1) << 15);
    g0[i] = e0 | (e1 << 16);
  }
  if constexpr (KM == 16) {
    const uint32_t m0 = (lane >> 5) ? 0u : ~0u;
    G[0] = make_uint4(g0[0] & m0, g0[1] & m0, g0[2] & m0, g0[3] & m0);
    G[1] = make_uint4(g0[0] & ~m0, g0[1] & ~m0, g0[2] & ~m0, g0[3] & ~m0);
    G[2] = G[0];
    G[3] = G[1];
  } else {
    const uint32_t hiflip = (lane >> 5) ? SGN : 0u;
    G[0] = make_uint4(g0[0], g0[1], g0[2], g0[3]);
    G[1] = make_uint4(g0[0] ^ hiflip, g0[1] ^ hiflip, g0[2] ^ hiflip, g0[3] ^ hiflip);
    G[2] = make_uint4(G[0].x ^ SGN, G[0].y ^ SGN, G[0].z ^ SGN, G[0].w ^ SGN);
    G[3] = make_uint4(G[1].x ^ SGN, G[1].y ^ SGN, G[1].z ^ SGN, G[1].w ^ SGN);
  }
}

// acc[nb] = 16 rows x columns 16nb + [0, 16) of x . blockdiag(H_KM), where x[ks] is the A
// fragment of columns 32ks + [0, 32) (lane l: row l%16, columns 32ks + 8(l/16) + [0, 8)).
template <class In, int KM, int NKS, int NNB>
__device__ inline void mma_rows(const uint4 (&x)[NKS], const uint4 (&G)[4], f32x4 (&acc)[NNB]) {
  constexpr int KB = KM >= 32 ? KM : 32;   // columns of one K block of the contraction
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      if ((32 * ks) / KB != (16 * nb) / KB) continue;   // outside the diagonal block
      const int sg = (KM == 16) ? 0 : (__builtin_popcount((2 * ks) & nb & (KM / 16 - 1)) & 1);
      acc[nb] = mma16<In>(x[ks], G[2 * sg + (nb & 1)], acc[nb]);
    }
  }
}

// Column strides 64 and 128 below min(K, LIM) (bits 2 and 3 of nb): H_2m = [[H_m, H_m],
// [H_m, -H_m]] as in-register butterflies between the 64-column blocks.
template <int K, int NNB, int LIM>
__device__ inline void mma_high_stages(f32x4 (&acc)[NNB]) {
#pragma unroll
  for (int hb = 4; hb <= 8; hb <<= 1) {
    if (16 * hb < K && 16 * hb < LIM && hb < NNB) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
        if ((nb & hb) == 0) {
          const f32x4 u = acc[nb], v = acc[nb + hb];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[nb][j] = u[j] + v[j];
            acc[nb + hb][j] = u[j] - v[j];
          }
        }
    }
  }
}

// 4 x 4 dword transpose across lane bits 2 and 3 (lanes 4m + i, m < 4, of each row of 16
// lanes): lane m's v[c] becomes lane c's v[m]. Bank-masked DPP moves, a lane keeping its own
// value where the mask leaves it out: lane ^ 8 is a rotation of the row by 8, lane ^ 4 a shift
// by four lanes in each direction.
template <int CTRL, int BANKS>
__device__ inline uint32_t dpp_take(uint32_t old, uint32_t src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, 0xF, BANKS, false);
}
__device__ inline void lane4_transpose(uint32_t& v0, uint32_t& v1, uint32_t& v2, uint32_t& v3) {
  // lane bit 3: positions 0, 1 of lanes 8-15 and 2, 3 of lanes 0-7 come from lane ^ 8
  const uint32_t a0 = dpp_take<0x128, 0xC>(v0, v2), a2 = dpp_take<0x128, 0x3>(v2, v0);
  const uint32_t a1 = dpp_take<0x128, 0xC>(v1, v3), a3 = dpp_take<0x128, 0x3>(v3, v1);
  // lane bit 2: positions 0, 2 of lanes with the bit set come from lane - 4 (row shift right),
  // positions 1, 3 of the others from lane + 4 (row shift left)
  v0 = dpp_take<0x114, 0xA>(a0, a1);
  v1 = dpp_take<0x104, 0x5>(a1, a0);
  v2 = dpp_take<0x114, 0xA>(a2, a3);
  v3 = dpp_take<0x104, 0x5>(a3, a2);
}

// 4 x 4 dword transpose across the lanes of a quad (lane p = lane & 3): lane p's v[c] becomes
// lane c's v[p]. Per lane bit, a quad permute fetches the partner's value and a select keeps it
// where the position's bit and the lane's bit differ.
__device__ inline void quad_transpose4(uint32_t (&v)[4], int p) {
  uint32_t n[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x = __builtin_amdgcn_mov_dpp(v[c ^ 2], 0x4E, 0xF, 0xF, false);   // lane ^ 2
    n[c] = (((c ^ p) >> 1) & 1) ? x : v[c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x = __builtin_amdgcn_mov_dpp(n[c ^ 1], 0xB1, 0xF, 0xF, false);   // lane ^ 1
    v[c] = ((c ^ p) & 1) ? x : n[c];
  }
}

// 4 x 4 byte transpose across the lanes of a quad: lane i of the quad holds bytes (row j, column
// 4m + i) for j < 4 and returns bytes (row i, column 4m + j).
__device__ inline uint32_t quad_byte_transpose(uint32_t d, int i) {
  const uint32_t selA = (i < 2) ? 0x05040100u : 0x03020706u;
  const uint32_t selB = (i & 1) ? 0x03070105u : 0x06020400u;
  const uint32_t p = __builtin_amdgcn_mov_dpp(d, 0x4E, 0xF, 0xF, false);   // lane ^ 2
  const uint32_t x = __builtin_amdgcn_perm(p, d, selA);
  const uint32_t q = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  return __builtin_amdgcn_perm(q, x, selB);
}

template <class In, int K, int OP>
__global__ __launch_bounds__(RM_THREADS, 2) void right_mma_kernel(ProArgs a) {
  if constexpr (In::bytes != 2 || K < 16) {
    return;
  } else {
    __shared__ __attribute__((aligned(16))) uint32_t tcode[RM_COLS * 16];   // [column][64 rows]
    __shared__ __attribute__((aligned(16))) uint32_t rcode[RM_ROWS * 64];   // [row][256 columns]
    __shared__ float red[32];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int n0 = lane & 15, lg = lane >> 4;
    const uint32_t nct = static_cast<uint32_t>(a.cols / RM_COLS);
    const uint32_t tiles = static_cast<uint32_t>(a.rows / RM_ROWS) * nct;   // < 2^31 (host checks)
    float sc = 0.0f, rinv = 0.0f;
    if constexpr (quant_op(OP)) {
      tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, sc, rinv);
      zero_side(a);
      if (blockIdx.x == 0 && t == 0) *a.scale_out = sc;
    }
    const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
    uint4 G[4];
    hfrags<In, (K < 64 ? K : 64)>(lane, G);
    const char* src = static_cast<const char*>(a.src);
    auto issue = [&](uint32_t tl, uint4 (&raw)[8]) {
      const uint32_t tp = a.rev ? tiles - 1u - tl : tl, tr = tp / nct;
      const int64_t row = static_cast<int64_t>(tr) * RM_ROWS + 16 * w + n0;
      const int64_t col = static_cast<int64_t>(tp - tr * nct) * RM_COLS + 8 * lg;
      const char* p = src + (row * a.cols + col) * 2;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) raw[ks] = *reinterpret_cast<const uint4*>(p + 64 * ks);
    };
    uint4 rawA[8], rawB[8];
    uint32_t tl = blockIdx.x;
    if (tl < tiles) issue(tl, rawA);
    float amax = 0.0f;
    auto body = [&](const uint32_t tl, const uint4 (&x)[8]) {
      f32x4 acc[16];
      mma_rows<In, (K < 64 ? K : 64), 8, 16>(x, G, acc);
      mma_high_stages<K, 16, 256>(acc);
      if constexpr (OP == OP_ABSMAX) {
#pragma unroll
        for (int nb = 0; nb < 16; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(acc[nb][j]));
      } else if constexpr (OP == OP_STORE) {
        // The rotated 64 x 256 tile in the input dtype goes through the two code buffers (rows
        // 0-31 in tcode, 32-63 in rcode; 512-byte rows), as packed column pairs: lanes n0 and
        // n0 ^ 1 hold columns c and c ^ 1 of rows 4lg + [0, 4); after a DPP swap the even lane
        // packs rows +0, +1 and the odd lane rows +3, +2. With the 16-byte chunk XOR-swizzled
        // by 4 ((row / 4) % 4) + 2 (row % 2), one instruction's 64 dword writes meet 64
        // distinct banks.
        const uint32_t tp = a.rev ? tiles - 1u - tl : tl, tr = tp / nct;
        const int64_t row0 = static_cast<int64_t>(tr) * RM_ROWS;
        const int64_t col0 = static_cast<int64_t>(tp - tr * nct) * RM_COLS;
        auto swz = [](int r) { return 4 * ((r >> 2) & 3) + 2 * (r & 1); };
        __syncthreads();   // the previous tile's readers of the buffers are done
        uint32_t* const half = (w >> 1) ? rcode : tcode;
        const bool odd = (n0 & 1) != 0;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
          float v[4], pv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = acc[nb][j];
            pv[j] = quad_xor1(v[j]);
          }
          const int cp = 8 * nb + (n0 >> 1);   // column pair (16nb + n0) / 2
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int rl = 16 * (w & 1) + 4 * lg + (odd ? 3 - jj : jj);
            const float lo = odd ? pv[3 - jj] : v[jj];
            const float hi = odd ? v[3 - jj] : pv[jj];
            half[rl * 128 + 4 * ((cp >> 2) ^ swz(rl)) + (cp & 3)] = In::pack2(lo, hi);
          }
        }
        __syncthreads();
        char* const dst = static_cast<char*>(a.dst);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int idx = 256 * p + t, row = idx >> 5, q = idx & 31, rl = row & 31;
          const uint32_t* hb = (row >> 5) ? rcode : tcode;
          *reinterpret_cast<uint4*>(dst + ((row0 + row) * a.cols + col0 + 8 * q) * 2) =
              *reinterpret_cast<const uint4*>(&hb[rl * 128 + 4 * (q ^ swz(rl))]);
        }
      } else {
        uint32_t d[16];   // rows 4lg + [0, 4) of column 16nb + n0
#pragma unroll
        for (int nb = 0; nb < 16; ++nb)
          d[nb] = quant4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3], rinv, lo, hi, (OP == OP_QUANT_F8));
        const uint32_t tp = a.rev ? tiles - 1u - tl : tl, tr = tp / nct;
        const int64_t row0 = static_cast<int64_t>(tr) * RM_ROWS;
        const int64_t col0 = static_cast<int64_t>(tp - tr * nct) * RM_COLS;
        __syncthreads();   // the previous tile's readers of the code tiles are done
        if (a.codes_t) {
#pragma unroll
          for (int nb = 0; nb < 16; ++nb) {
            const int c = 16 * nb + n0;
            tcode[c * 16 + ((4 * w + lg) ^ (4 * ((c >> 2) & 3)))] = d[nb];
          }
        }
        if (a.codes) {
          const int i = n0 & 3, m = n0 >> 2, row = 16 * w + 4 * lg + i;
#pragma unroll
          for (int nb = 0; nb < 16; ++nb)
            rcode[row * 64 + ((4 * nb + m) ^ (4 * (row & 15)))] = quad_byte_transpose(d[nb], i);
        }
        __syncthreads();
        if (a.codes_t) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int idx = 256 * p + t, c = idx >> 2, q = idx & 3;
            *reinterpret_cast<uint4*>(a.codes_t + (col0 + c) * a.ld_t + row0 + 16 * q) =
                *reinterpret_cast<const uint4*>(&tcode[c * 16 + 4 * (q ^ ((c >> 2) & 3))]);
          }
        }
        if (a.codes) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int idx = 256 * p + t, row = idx >> 4, cc = idx & 15;
            *reinterpret_cast<uint4*>(a.codes + (row0 + row) * a.ld + col0 + 16 * cc) =
                *reinterpret_cast<const uint4*>(&rcode[row * 64 + 4 * (cc ^ (row & 15))]);
          }
        }
      }
    };
    while (tl < tiles) {
      const uint32_t t1 = tl + gridDim.x;
      issue(t1 < tiles ? t1 : tl, rawB);   // unconditional: the last re-reads
      body(tl, rawA);
      if (t1 >= tiles) break;
      const uint32_t t2 = t1 + gridDim.x;
      issue(t2 < tiles ? t2 : t1, rawA);
      body(t1, rawB);
      tl = t2;
    }
    if constexpr (OP == OP_ABSMAX) {
      amax = block_max(amax, red);
      if (t == 0) a.partials[blockIdx.x] = amax;
    }
  }
}

// ================================================================ left rotation
constexpr int LT_THREADS = 256, LT_ELEMS = 16384;

template <int KL> struct LeftShape {
  static constexpr int TR = KL > 64 ? KL : 64;   // tile rows: whole k-blocks, >= 64
  static constexpr int TC = LT_ELEMS / TR;       // tile columns
  static constexpr int P = TR / 64;              // lanes sharing a column (1, 2 or 4)
  static constexpr int PITCH = TC + 4;           // LDS row pitch (floats)
};

template <class In, int K, int OP>
__global__ __launch_bounds__(LT_THREADS) void left_kernel(ProArgs a) {
  using S = LeftShape<K>;
  constexpr int TR = S::TR, TC = S::TC, P = S::P, PITCH = S::PITCH;
  __shared__ __attribute__((aligned(16))) float tile[TR * PITCH];
  __shared__ float red[32];
  int8_t* bcodes = reinterpret_cast<int8_t*>(tile);   // reused for row-major codes: TR x (TC+16)
  constexpr int BP = TC + 16;
  const int t = threadIdx.x, lane = t & 63;
  const int c = t / P, p = t % P;                     // column, 64-row part
  const int64_t nrt = (a.rows + TR - 1) / TR, nct = (a.cols + TC - 1) / TC;
  const int64_t tiles = nrt * nct;
  float sc = 0.0f, rinv = 0.0f;
  if constexpr (quant_op(OP)) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, sc, rinv);
    zero_side(a);
    if (blockIdx.x == 0 && t == 0) *a.scale_out = sc;
  }
  const int64_t rpad = (a.rows + 15) / 16 * 16, cpad = (a.cols + 15) / 16 * 16;
  auto slot = [](int row, int col) { return row * PITCH + (col ^ ((64 / P) * (row >> 6))); };
  float amax = 0.0f;
  for (int64_t tl = blockIdx.x; tl < tiles; tl += gridDim.x) {
    const int64_t row0 = (tl / nct) * TR, col0 = (tl % nct) * TC;
    __syncthreads();
    // stage the tile as fp32: 8 consecutive columns per thread per step
    for (int q = t; q < TR * TC / 8; q += LT_THREADS) {
      const int row = q / (TC / 8), cc = 8 * (q % (TC / 8));
      const int64_t grow = row0 + row, gc = col0 + cc;
      float f[8];
      if (grow < a.rows && gc < a.cols) {
        const char* rp = static_cast<const char*>(a.src) + grow * a.cols * In::bytes;
        if (a.vec && gc + 8 <= a.cols) {
          if constexpr (In::bytes == 4) {
            const float4 x0 = *reinterpret_cast<const float4*>(rp + 4 * gc);
            const float4 x1 = *reinterpret_cast<const float4*>(rp + 4 * gc + 16);
            f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
            f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
          } else {
            const uint4 u = *reinterpret_cast<const uint4*>(rp + 2 * gc);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              f[2 * j] = In::from_bits(static_cast<uint16_t>(w[j] & 0xFFFFu));
              f[2 * j + 1] = In::from_bits(static_cast<uint16_t>(w[j] >> 16));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = (gc + j < a.cols) ? In::load(rp, gc + j) : 0.0f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = 0.0f;
      }
      *reinterpret_cast<float4*>(&tile[slot(row, cc)]) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(&tile[slot(row, cc + 4)]) = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
    float v[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = tile[slot(64 * p + i, c)];
    fwht_inreg<K, 64>(v);
    if constexpr (K > 64) quad_stage<64>(v, lane, 1);
    if constexpr (K > 128) quad_stage<64>(v, lane, 2);
    const int64_t gcol = col0 + c;
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
    } else {
      // transposed codes: 64 consecutive tokens of column gcol
      if (a.codes_t && gcol < a.cols) {
        int8_t* dst = a.codes_t + gcol * a.ld_t + row0 + 64 * p;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (row0 + 64 * p + 16 * q < rpad) *reinterpret_cast<uint4*>(dst + 16 * q) = pack16(v, 16 * q, rinv, a.qp, (OP == OP_QUANT_F8), static_cast<float>(a.fgrid), a.qmaxf);
      }
      if (a.codes) {
        __syncthreads();   // the fp32 tile is dead: reuse it for the byte transpose
#pragma unroll
        for (int i = 0; i < 64; ++i)
          bcodes[(64 * p + i) * BP + c] = static_cast<int8_t>(quant_byte(v[i], rinv, a.qp, (OP == OP_QUANT_F8), static_cast<float>(a.fgrid), a.qmaxf));
        __syncthreads();
        for (int q = t; q < TR * TC / 16; q += LT_THREADS) {
          const int row = q / (TC / 16), cc = 16 * (q % (TC / 16));
          const int64_t grow = row0 + row, gc = col0 + cc;
          if (grow < a.rows && gc < cpad)
            *reinterpret_cast<uint4*>(a.codes + grow * a.ld + gc) =
                *reinterpret_cast<const uint4*>(&bcodes[row * BP + cc]);
        }
      }
    }
  }
  if constexpr (OP == OP_ABSMAX) {
    amax = block_max(amax, red);
    if (t == 0) a.partials[blockIdx.x] = amax;
  }
}

// ================================================================ left rotation, full tiles
// Used when rows are whole 256-row tiles and columns whole 64-column tiles of 16-bit inputs
// with 16-byte aligned rows. Persistent workgroups walk 256 x 64 tiles; the raw bytes of the
// next tile are loaded into registers before the current tile is worked on. A tile is staged
// in LDS as fp32 (column index XOR-swizzled by 16 * (row / 64), so the column reads below are
// conflict-free); thread (column c, part p) then takes the 64 consecutive tokens 64 p + [0, 64)
// of column c: token strides 1..32 are in-register butterflies, 64 and 128 are one-instruction
// quad DPP stages (v_fmac_dpp, the upper lane's sign folded into the quantizer).
// Transposed codes leave directly as 64 consecutive tokens; row-major codes are transposed as
// 4 x 4 byte blocks across the lanes of four neighbouring columns (DPP + v_perm) and
// assembled in LDS into 64-byte rows.
constexpr int LF_ROWS = 256, LF_COLS = 64, LF_THREADS = 256, LF_PITCH = LF_COLS + 4, LF_GRID = 512;

// Dword slot swizzle of the 256 x 64-byte code tile: a row's sixteen 4-column groups are
// permuted so that both the transposed writes (rows 64 p + 4 g + b) and the row reads meet
// distinct banks.
__device__ inline int lf_swz(int row) { return (row & 15) ^ ((row >> 4) & 3) ^ (4 * ((row >> 6) & 3)); }

__host__ __device__ inline bool left_fast_ok(int64_t rows, int64_t cols, bool vec, int in_bytes) {
  return vec && in_bytes == 2 && rows > 0 && cols > 0 && rows % LF_ROWS == 0 && cols % LF_COLS == 0 &&
         (rows / LF_ROWS) * (cols / LF_COLS) < (int64_t(1) << 31);
}

template <class In, int K, int OP>
__global__ __launch_bounds__(LF_THREADS, 2) void left_fast_kernel(ProArgs a) {
  if constexpr (In::bytes != 2) {
    return;   // never launched: left_fast_ok admits 16-bit inputs only
  } else {
  __shared__ __attribute__((aligned(16))) float tile[LF_ROWS * LF_PITCH];
  __shared__ float red[32];
  const int t = threadIdx.x, lane = t & 63;
  const int c = t >> 2, p = t & 3;              // column of the tile, 64-token part
  const uint32_t nct = static_cast<uint32_t>(a.cols / LF_COLS);
  const uint32_t tiles = static_cast<uint32_t>(a.rows / LF_ROWS) * nct;   // < 2^31 (host checks)
  float sc = 0.0f, rinv = 0.0f;
  if constexpr (quant_op(OP)) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, sc, rinv);
    zero_side(a);
    if (blockIdx.x == 0 && t == 0) *a.scale_out = sc;
  }
  constexpr int XMASK = K > 128 ? 3 : (K > 64 ? 1 : 0);
  const float rr = (__builtin_popcount(lane & XMASK) & 1) ? -rinv : rinv;
  const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
  const float sg1 = (lane & 1) ? -1.0f : 1.0f, sg2 = (lane & 2) ? -1.0f : 1.0f;
  const char* src = static_cast<const char*>(a.src);
  // global loads: eight 16-byte chunks per thread, row 32 q + t / 8, columns 8 (t % 8) + [0, 8)
  const int lr = t >> 3, lc = 8 * (t & 7);
  auto issue = [&](uint32_t tl, uint4 (&raw)[8]) {
    const uint32_t tr = tl / nct;
    const int64_t row = static_cast<int64_t>(tr) * LF_ROWS + lr;
    const int64_t col = static_cast<int64_t>(tl - tr * nct) * LF_COLS + lc;
    const char* q0 = src + (row * a.cols + col) * 2;
#pragma unroll
    for (int q = 0; q < 8; ++q) raw[q] = *reinterpret_cast<const uint4*>(q0 + static_cast<int64_t>(32 * q) * a.cols * 2);
  };
  const int rbase = 64 * p * LF_PITCH + (c ^ (16 * p));   // this thread's column in part p
  uint4 rawA[8], rawB[8];
  uint32_t tl = blockIdx.x;
  if (tl < tiles) issue(tl, rawA);
  float amax = 0.0f;
  // one tile in registers while the next one loads: two register sets, alternating
  auto body = [&](const uint32_t tl, const uint4 (&cur)[8]) {
    __syncthreads();   // the previous tile's readers of the LDS tile are done
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 32 * q + lr;
      const uint32_t w[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = In::from_bits(static_cast<uint16_t>(w[j] & 0xFFFFu));
        f[2 * j + 1] = In::from_bits(static_cast<uint16_t>(w[j] >> 16));
      }
      float* d = &tile[row * LF_PITCH + (lc ^ (16 * (row >> 6)))];
      *reinterpret_cast<float4*>(d) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
    float v[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = tile[rbase + i * LF_PITCH];
    fwht_inreg<K, 64>(v);
    if constexpr (K > 64) xstage_signed<1>(v, sg1);
    if constexpr (K > 128) xstage_signed<2>(v, sg2);
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
    } else {
      uint32_t d[16];   // d[g]: tokens 64 p + 4 g + [0, 4) of column c
#pragma unroll
      for (int g = 0; g < 16; ++g)
        d[g] = quant4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], rr, lo, hi, (OP == OP_QUANT_F8));
      const uint32_t tr = tl / nct;
      const int64_t row0 = static_cast<int64_t>(tr) * LF_ROWS;
      const int64_t col0 = static_cast<int64_t>(tl - tr * nct) * LF_COLS;
      if (a.codes_t) {
        uint4* dst = reinterpret_cast<uint4*>(a.codes_t + (col0 + c) * a.ld_t + row0 + 64 * p);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = make_uint4(d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]);
      }
      if (a.codes) {
        // 4 x 4 byte transpose across the lanes of columns 4m .. 4m+3 (lane bits 2, 3): lane
        // b = (lane >> 2) & 3 ends with the codes of columns 4m .. 4m+3 of token 4 g + b
        const int b = (lane >> 2) & 3;
        const uint32_t selA = (b < 2) ? 0x05040100u : 0x03020706u;
        const uint32_t selB = (b & 1) ? 0x03070105u : 0x06020400u;
        uint32_t* ct = reinterpret_cast<uint32_t*>(tile);   // code tile: 256 rows x 64 bytes
        __syncthreads();   // every thread has read its column of the fp32 tile
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const uint32_t pv = __builtin_amdgcn_mov_dpp(d[g], 0x128, 0xF, 0xF, false);   // lane ^ 8
          const uint32_t x = __builtin_amdgcn_perm(pv, d[g], selA);
          uint32_t q = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0x5, false);           // lane + 4
          q = __builtin_amdgcn_update_dpp(q, x, 0x114, 0xF, 0xA, false);                     // lane - 4
          const uint32_t e = __builtin_amdgcn_perm(q, x, selB);
          const int row = 64 * p + 4 * g + b;
          ct[row * 16 + ((c >> 2) ^ lf_swz(row))] = e;
        }
        __syncthreads();
        // thread t: tile row t, 64 bytes
        uint32_t e[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) e[j] = ct[t * 16 + (j ^ lf_swz(t))];
        uint4* dst = reinterpret_cast<uint4*>(a.codes + (row0 + t) * a.ld + col0);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = make_uint4(e[4 * j], e[4 * j + 1], e[4 * j + 2], e[4 * j + 3]);
      }
    }
    };
  while (tl < tiles) {
    const uint32_t t1 = tl + gridDim.x;
    issue(t1 < tiles ? t1 : tl, rawB);   // unconditional: the last re-reads
    body(tl, rawA);
    if (t1 >= tiles) break;
    const uint32_t t2 = t1 + gridDim.x;
    issue(t2 < tiles ? t2 : t1, rawA);
    body(t1, rawB);
    tl = t2;
  }
  if constexpr (OP == OP_ABSMAX) {
    amax = block_max(amax, red);
    if (t == 0) a.partials[blockIdx.x] = amax;
  }
  }
}

// ================================================================ left rotation on the matrix cores
// Token-axis rotation of 16-bit tensors of whole 256 x 64 tiles (dY under HALO-2) as the product
// blockdiag(H_k) . Y_tile on the matrix cores. H is symmetric, so its A fragments are the B
// fragments of mma_rows with the output block nb read as the output row block mb. The tile is
// staged in LDS as raw 16-bit values, rows of 128 bytes whose 16-byte chunk c sits at
// c ^ 2((row / 8) % 4); wave w takes columns 16w + [0, 16) and builds its B fragments (lane l:
// column l%16, rows 32ks + 8(l/16) + [0, 8)) from 16-bit reads that meet distinct banks. The output
// (lane l: rows 16mb + 4(l/16) + [0, 4) of column 16w + l%16) leaves as in right_mma_kernel:
// dwords of the transposed codes directly, row-major codes through the quad byte transpose, both
// through XOR-swizzled LDS tiles with conflict-free dword writes and 16-byte reads.
constexpr int LM_ROWS = 256, LM_COLS = 64, LM_THREADS = 256, LM_GRID = 512;

__host__ __device__ inline bool left_mma_ok(int64_t rows, int64_t cols, bool vec, int in_bytes,
                                            int k) {
  return k >= 16 && k <= LM_ROWS && left_fast_ok(rows, cols, vec, in_bytes);
}

// acc[mb] = output rows 16mb + [0, 16) of blockdiag(H_KM) . y for the wave's 16 columns, where
// y[ks] is the B fragment of rows 32ks + [0, 32).
template <class In, int KM, int NKS, int NMB>
__device__ inline void mma_cols(const uint4 (&G)[4], const uint4 (&y)[NKS], f32x4 (&acc)[NMB]) {
  constexpr int KB = KM >= 32 ? KM : 32;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if ((32 * ks) / KB != (16 * mb) / KB) continue;
      const int sg = (KM == 16) ? 0 : (__builtin_popcount((2 * ks) & mb & (KM / 16 - 1)) & 1);
      acc[mb] = mma16<In>(G[2 * sg + (mb & 1)], y[ks], acc[mb]);
    }
  }
}

template <class In, int K, int OP>
__global__ __launch_bounds__(LM_THREADS, 2) void left_mma_kernel(ProArgs a) {
  if constexpr (In::bytes != 2 || K < 16) {
    return;
  } else {
    __shared__ __attribute__((aligned(16))) uint4 tile[LM_ROWS * 8];         // [row][8 chunks]
    __shared__ __attribute__((aligned(16))) uint32_t tcode[LM_COLS * 64];    // [column][256 rows]
    __shared__ __attribute__((aligned(16))) uint32_t rcode[LM_ROWS * 16];    // [row][64 columns]
    __shared__ float red[32];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int n0 = lane & 15, lg = lane >> 4;
    const uint32_t nct = static_cast<uint32_t>(a.cols / LM_COLS);
    const uint32_t tiles = static_cast<uint32_t>(a.rows / LM_ROWS) * nct;   // < 2^31 (host checks)
    float sc = 0.0f, rinv = 0.0f;
    if constexpr (quant_op(OP)) {
      tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, sc, rinv);
      zero_side(a);
      if (blockIdx.x == 0 && t == 0) *a.scale_out = sc;
    }
    const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
    uint4 G[4];
    hfrags<In, (K < 64 ? K : 64)>(lane, G);
    const char* src = static_cast<const char*>(a.src);
    // thread t loads chunks 256p + t: row (256p + t) / 8, 8 columns from 8((256p + t) % 8)
    auto issue = [&](uint32_t tl, uint4 (&raw)[8]) {
      const uint32_t tp = a.rev ? tiles - 1u - tl : tl, tr = tp / nct;
      const int64_t row = static_cast<int64_t>(tr) * LM_ROWS + (t >> 3);
      const int64_t col = static_cast<int64_t>(tp - tr * nct) * LM_COLS + 8 * (t & 7);
      const uint4* p = reinterpret_cast<const uint4*>(src + (row * a.cols + col) * 2);
      const int64_t step = a.cols * 4;   // 32 rows, in uint4
#pragma unroll
      for (int q = 0; q < 8; ++q) raw[q] = p[q * step];
    };
    const uint16_t* th = reinterpret_cast<const uint16_t*>(tile);
    uint4 rawA[8], rawB[8];
    uint32_t tl = blockIdx.x;
    if (tl < tiles) issue(tl, rawA);
    float amax = 0.0f;
    auto body = [&](const uint32_t tl, const uint4 (&raw)[8]) {
      __syncthreads();   // the previous tile's readers of the LDS tiles are done
      {
        // chunk q of this thread: row 32q + t/8 (same (row / 8) % 4 for every q), chunk t % 8
        const int rr = t >> 3;
        uint4* tp = tile + rr * 8 + ((t & 7) ^ (2 * ((rr >> 3) & 3)));
        const uint4 r0 = raw[0], r1 = raw[1], r2 = raw[2], r3 = raw[3];
        const uint4 r4 = raw[4], r5 = raw[5], r6 = raw[6], r7 = raw[7];
        tp[0] = r0; tp[256] = r1; tp[512] = r2; tp[768] = r3;
        tp[1024] = r4; tp[1280] = r5; tp[1536] = r6; tp[1792] = r7;
      }
      __syncthreads();
      uint4 y[8];
      {
        const int c = 2 * w + (n0 >> 3), e = n0 & 7;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int r0 = 32 * ks + 8 * lg;   // (r0 / 8) % 4 == lg
          const uint16_t* p = th + r0 * 64 + 8 * (c ^ (2 * lg)) + e;
          uint32_t v[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            v[jj] = static_cast<uint32_t>(p[(2 * jj) * 64]) | (static_cast<uint32_t>(p[(2 * jj + 1) * 64]) << 16);
          y[ks] = make_uint4(v[0], v[1], v[2], v[3]);
        }
      }
      f32x4 acc[16];
      mma_cols<In, (K < 64 ? K : 64), 8, 16>(G, y, acc);
      mma_high_stages<K, 16, 256>(acc);
      if constexpr (OP == OP_ABSMAX) {
#pragma unroll
        for (int mb = 0; mb < 16; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(acc[mb][j]));
      } else if constexpr (OP == OP_STORE) {
        // The rotated tile in the input dtype goes back through the raw buffer (every wave has
        // read its fragments once all pass the barrier), row-major with 128-byte rows. Lanes
        // n0 and n0 ^ 1 hold columns c and c ^ 1 of rows 16mb + 4lg + [0, 4); after a DPP swap
        // the even lane packs rows +0, +1 and the odd lane rows +3, +2 of the column pair, so
        // one instruction's rows alternate in parity and, with the 16-byte chunk XOR-swizzled
        // by 2 ((row / 4) % 4), its 64 dword writes meet 64 distinct banks.
        __syncthreads();
        uint32_t* const to = reinterpret_cast<uint32_t*>(tile);
        const bool odd = (n0 & 1) != 0;
        const int cp = 8 * w + (n0 >> 1);   // column pair (16w + n0) / 2
#pragma unroll
        for (int mb = 0; mb < 16; ++mb) {
          float v[4], pv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = acc[mb][j];
            pv[j] = quad_xor1(v[j]);
          }
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int row = 16 * mb + 4 * lg + (odd ? 3 - jj : jj);
            const float lo = odd ? pv[3 - jj] : v[jj];
            const float hi = odd ? v[3 - jj] : pv[jj];
            to[row * 32 + 4 * ((cp >> 2) ^ (2 * ((row >> 2) & 3))) + (cp & 3)] = In::pack2(lo, hi);
          }
        }
        __syncthreads();
        const uint32_t tp = a.rev ? tiles - 1u - tl : tl, tr = tp / nct;
        const int64_t row0 = static_cast<int64_t>(tr) * LM_ROWS;
        const int64_t col0 = static_cast<int64_t>(tp - tr * nct) * LM_COLS;
        char* const dst = static_cast<char*>(a.dst);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int idx = 256 * p + t, row = idx >> 3, q = idx & 7;
          *reinterpret_cast<uint4*>(dst + ((row0 + row) * a.cols + col0 + 8 * q) * 2) =
              tile[row * 8 + (q ^ (2 * ((row >> 2) & 3)))];
        }
      } else {
        uint32_t d[16];   // rows 16mb + 4lg + [0, 4) of column 16w + n0
#pragma unroll
        for (int mb = 0; mb < 16; ++mb)
          d[mb] = quant4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3], rinv, lo, hi, (OP == OP_QUANT_F8));
        const uint32_t tp = a.rev ? tiles - 1u - tl : tl, tr = tp / nct;
        const int64_t row0 = static_cast<int64_t>(tr) * LM_ROWS;
        const int64_t col0 = static_cast<int64_t>(tp - tr * nct) * LM_COLS;
        if (a.codes_t) {
          const int c = 16 * w + n0;
#pragma unroll
          for (int mb = 0; mb < 16; ++mb) tcode[c * 64 + ((4 * mb + lg) ^ (4 * n0))] = d[mb];
        }
        if (a.codes) {
          const int i = n0 & 3, m = n0 >> 2;
#pragma unroll
          for (int mb = 0; mb < 16; ++mb) {
            const int row = 16 * mb + 4 * lg + i;   // (row / 4) % 4 == lg
            rcode[row * 16 + ((4 * w + m) ^ (4 * lg))] = quad_byte_transpose(d[mb], i);
          }
        }
        __syncthreads();
        if (a.codes_t) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int idx = 256 * p + t, c = idx >> 4, q = idx & 15;
            *reinterpret_cast<uint4*>(a.codes_t + (col0 + c) * a.ld_t + row0 + 16 * q) =
                *reinterpret_cast<const uint4*>(&tcode[c * 64 + 4 * (q ^ (c & 15))]);
          }
        }
        if (a.codes) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int idx = 256 * p + t, row = idx >> 2, q = idx & 3;
            *reinterpret_cast<uint4*>(a.codes + (row0 + row) * a.ld + col0 + 16 * q) =
                *reinterpret_cast<const uint4*>(&rcode[row * 16 + 4 * (q ^ ((row >> 2) & 3))]);
          }
        }
      }
    };
    while (tl < tiles) {
      const uint32_t t1 = tl + gridDim.x;
      issue(t1 < tiles ? t1 : tl, rawB);   // unconditional: the last re-reads
      body(tl, rawA);
      if (t1 >= tiles) break;
      const uint32_t t2 = t1 + gridDim.x;
      issue(t2 < tiles ? t2 : t1, rawA);
      body(t1, rawB);
      tl = t2;
    }
    if constexpr (OP == OP_ABSMAX) {
      amax = block_max(amax, red);
      if (t == 0) a.partials[blockIdx.x] = amax;
    }
  }
}

// ================================================================ both (X under HALO-2)
constexpr int BT = 256, BT_THREADS = 512, BT_HALF = 128, BT_PITCH = BT_HALF + 4;

// 64 consecutive elements starting at c0 of a row with n valid elements, with the stride-1
// butterfly already applied (fp16 / bf16 pairs go through v_dot2 with (1, 1) and (1, -1)).
template <class T>
__device__ inline void load64_s1(const void* row, int64_t c0, int64_t n, bool vec, float (&v)[64]) {
  if constexpr (T::bytes == 2) {
    if (vec && c0 + 64 <= n) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + c0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 u = p[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (T::is_bf16) {
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            const b2 x = __builtin_bit_cast(b2, w[j]);
            v[8 * q + 2 * j] = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(b2, 0x3F803F80u), 0.0f, false);
            v[8 * q + 2 * j + 1] = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(b2, 0xBF803F80u), 0.0f, false);
          } else {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            const h2 x = __builtin_bit_cast(h2, w[j]);
            v[8 * q + 2 * j] = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(h2, 0x3C003C00u), 0.0f, false);
            v[8 * q + 2 * j + 1] = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(h2, 0xBC003C00u), 0.0f, false);
          }
        }
      }
      return;
    }
  }
  load64<T>(row, c0, n, vec, v);
  fwht_inreg<2, 64>(v);
}

// f64 butterfly across the lanes of a quad (m = 1 or 2), as quad_stage.
template <int M, int N>
__device__ inline void quad_stage_f64(double (&u)[N], int lane) {
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;
  const double sgn = (lane & M) ? -1.0 : 1.0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint64_t b = __builtin_bit_cast(uint64_t, u[i]);
    const int lo = static_cast<int>(b), hi = static_cast<int>(b >> 32);
    const int plo = __builtin_amdgcn_mov_dpp(lo, ctrl, 0xF, 0xF, false);
    const int phi = __builtin_amdgcn_mov_dpp(hi, ctrl, 0xF, 0xF, false);
    const double p = __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(phi)) << 32) |
                                                    static_cast<uint32_t>(plo));
    u[i] = __builtin_fma(u[i], sgn, p);
    if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);   // bound the live DPP temporaries
  }
}

// The token-axis phase of the two-sided transform (B (X B)) sums the fp32 values of X B in
// fp32 butterflies: log2 k rounded additions per value, within the code and output tolerances
// (a code may move by one step where B X B lies within that rounding of a midpoint). With
// TokenT = double the sums are exact and B X B is rounded once.
using TokenT = float;

template <int M, int N>
__device__ inline void quad_stage_tok(float (&u)[N], int lane) { quad_stage<N>(u, lane, M); }
template <int M, int N>
__device__ inline void quad_stage_tok(double (&u)[N], int lane) { quad_stage_f64<M, N>(u, lane); }

// Work items of both_kernel: 128-column halves of 256 x 256 tiles. The two halves of a tile are
// 8 items apart, so that they run on one XCD and the second read of the tile hits its L2.
__host__ __device__ inline int64_t both_items(int64_t rows, int64_t cols) {
  return 2 * ((rows + BT - 1) / BT) * ((cols + BT - 1) / BT);
}

// Per item: the tile rows rotated along the feature axis (X B in fp32, exact for 16-bit inputs;
// with k = 256 both halves of a row are needed, otherwise only the item's own half is read) give
// the row-major codes of X B; the item's half of X B is then staged through LDS (16-column
// blocks XOR-swizzled by row / 64 and the 64-column half, so both the row-wise 16-byte writes
// and the column reads are conflict-free) and rotated along the token axis in TokenT before
// its scale and codes are taken.
template <class In, int K, int OP>
__global__ __launch_bounds__(BT_THREADS) void both_kernel(ProArgs a) {
  __shared__ __attribute__((aligned(16))) float half[BT * BT_PITCH];
  __shared__ float red[32];
  const int t = threadIdx.x, lane = t & 63;
  const int r = t >> 1, s2 = t & 1;      // row phase: row r, columns 64*s2 + [0, 64) of a half
  const int cp = t >> 2, pp = t & 3;     // column phase: column cp of the half, rows 64*pp + [0, 64)
  const int64_t nct = (a.cols + BT - 1) / BT;
  const int64_t items = both_items(a.rows, a.cols);
  float s1 = 0.0f, r1 = 0.0f, sc2 = 0.0f, r2 = 0.0f;
  if constexpr (quant_op(OP)) {
    tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, s1, r1);
    tensor_scale(a.part_in2, a.nparts, a.step2, a.qmaxf, red, sc2, r2);
    zero_side(a);
    if (blockIdx.x == 0 && t == 0) {
      *a.scale_out = s1;
      *a.scale_out2 = sc2;
    }
  }
  const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
  const int64_t rpad = (a.rows + 15) / 16 * 16, cpad = (a.cols + 15) / 16 * 16;
  const char* src = static_cast<const char*>(a.src);
  float amax1 = 0.0f, amax2 = 0.0f;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t full = items / 16 * 16;
    int64_t tl;
    int h;
    if (it < full) {
      tl = (it / 16) * 8 + (it % 8);
      h = static_cast<int>((it / 8) & 1);
    } else {
      tl = full / 2 + (it - full) / 2;
      h = static_cast<int>((it - full) & 1);
    }
    const int64_t row0 = (tl / nct) * BT, col0 = (tl % nct) * BT;
    const int64_t grow = row0 + r;
    const bool rin = grow < a.rows;
    const char* rowp = src + grow * a.cols * In::bytes;
    // ---- row phase: this half of X B for row r, columns 64*s2 + [0, 64)
    float w[64];
    const int64_t gc = col0 + BT_HALF * h + 64 * s2;
    if constexpr (K > 128) {
      float v[2][64];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int64_t c = col0 + BT_HALF * hh + 64 * s2;
        if (rin && c < a.cols) {
          load64_s1<In>(rowp, c, a.cols, a.vec, v[hh]);
        } else {
#pragma unroll
          for (int j = 0; j < 64; ++j) v[hh][j] = 0.0f;
        }
        fwht_from<2, K, 64>(v[hh]);
        quad_stage<64>(v[hh], lane, 1);
      }
      const float sg = h ? -1.0f : 1.0f;   // stride 128: the lower half keeps x + y, the upper x - y
#pragma unroll
      for (int j = 0; j < 64; ++j) w[j] = __builtin_fmaf(v[1][j], sg, v[0][j]);
    } else {
      if (rin && gc < a.cols) {
        load64_s1<In>(rowp, gc, a.cols, a.vec, w);
      } else {
#pragma unroll
        for (int j = 0; j < 64; ++j) w[j] = 0.0f;
      }
      fwht_from<2, K, 64>(w);
      if constexpr (K > 64) quad_stage<64>(w, lane, 1);
    }
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int j = 0; j < 64; ++j) amax1 = fmaxf(amax1, fabsf(w[j]));
    } else if (a.codes && rin) {
      int8_t* dst = a.codes + grow * a.ld + gc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (gc + 16 * q < cpad) {
          uint32_t x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 16 * q + 4 * j;
            x[j] = quant4(w[i], w[i + 1], w[i + 2], w[i + 3], r1, lo, hi, (OP == OP_QUANT_F8));
          }
          *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(x[0], x[1], x[2], x[3]);
        }
      }
    }
    // ---- column phase: the token-axis rotation of this half, in TokenT
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      float* dst = &half[r * BT_PITCH + ((64 * s2 + 16 * jb) ^ (16 * (r >> 6)) ^ (32 * s2))];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 4 * q) =
            make_float4(w[16 * jb + 4 * q], w[16 * jb + 4 * q + 1], w[16 * jb + 4 * q + 2], w[16 * jb + 4 * q + 3]);
    }
    __syncthreads();
    TokenT u[64];
    const float* col = &half[64 * pp * BT_PITCH + (cp ^ (16 * pp) ^ (32 * (cp >> 6)))];
#pragma unroll
    for (int i = 0; i < 64; ++i) u[i] = static_cast<TokenT>(col[i * BT_PITCH]);
    fwht_from<1, K, 64>(u);
    if constexpr (K > 64) quad_stage_tok<1, 64>(u, lane);
    if constexpr (K > 128) quad_stage_tok<2, 64>(u, lane);
    const int64_t gcol = col0 + BT_HALF * h + cp;
    if constexpr (OP == OP_ABSMAX) {
#pragma unroll
      for (int i = 0; i < 64; ++i) amax2 = fmaxf(amax2, fabsf(static_cast<float>(u[i])));
    } else if (gcol < a.cols) {
      int8_t* dst = a.codes_t + gcol * a.ld_t + row0 + 64 * pp;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (row0 + 64 * pp + 16 * q < rpad) {
          uint32_t x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 16 * q + 4 * j;
            x[j] = quant4(static_cast<float>(u[i]), static_cast<float>(u[i + 1]),
                          static_cast<float>(u[i + 2]), static_cast<float>(u[i + 3]), r2, lo, hi,
                          (OP == OP_QUANT_F8));
          }
          *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(x[0], x[1], x[2], x[3]);
        }
      }
    }
  }
  if constexpr (OP == OP_ABSMAX) {
    amax1 = block_max(amax1, red);
    amax2 = block_max(amax2, red);
    if (t == 0) {
      a.partials[blockIdx.x] = amax1;
      a.partials[gridDim.x + blockIdx.x] = amax2;
    }
  }
}

// ================================================================ both, row phase on the matrix cores
// X under HALO-2 for 16-bit inputs and whole 256 x 256 tiles. Work items as both_kernel (the
// 128-column half h of a tile, halves 8 items apart). Row phase: wave w rotates tile rows
// 32w + [0, 32) as two 16-row blocks on the matrix cores (mma_rows; for k = 256 all sixteen
// 16-column blocks of the row, the stride-64 butterfly on both halves, then the stride-128 stage
// for this half only, lower half x + y, upper half x - y). Its output (lane l: rows 4(l/16) + [0, 4)
// of column 16nb + l%16) gives the row-major codes of X B through the quad byte transpose, and goes
// to LDS column-major as one 16-byte write per lane and block: the half tile is
// [128 columns][256 rows] fp32, 16-byte row chunk c4 of column c stored at chunk
// c4 ^ (c % 16) ^ 4((c4 / 16) % 4), so the writes (16 columns per 16 lanes) and the column
// phase's reads (4 columns x 4 row quarters per 16 lanes) are conflict-free. Column phase as
// both_kernel: lane (column cp, quarter pp) rotates rows 64pp + [0, 64) in TokenT.
constexpr int BM_THREADS = 512;

__host__ __device__ inline bool both_mma_ok(int64_t rows, int64_t cols, bool vec, int in_bytes,
                                            int k) {
  return vec && in_bytes == 2 && k >= 16 && k <= BT && rows > 0 && cols > 0 && rows % BT == 0 &&
         cols % BT == 0 && cols <= (int64_t(1) << 22);   // 256 rows stay 32-bit addressable
}

__device__ inline int bm_chunk(int c, int c4) { return c4 ^ (c & 15) ^ (4 * ((c4 >> 4) & 3)); }

// PIPE (a workgroup has several items): the item's raw 16-bit rows (all 256 columns for k = 256,
// else the item's 128) are brought into the half-tile buffer by direct-to-LDS buffer loads,
// issued as soon as the previous item's column phase has read its values out of LDS, so they
// land while that item's token-axis rotation runs. Rows of RAWB bytes, 16-byte chunk c of row r at
// c ^ (r % 16): the fragment reads of 16 consecutive rows meet distinct bank groups. Each wave
// reads its A fragments from there, and after a barrier the buffer takes the fp32 half tile.
template <class In, int K, int OP, bool PIPE>
__device__ inline void both_mma_body(const ProArgs& a) {
  {
    __shared__ __attribute__((aligned(16))) float half[BT_HALF * BT];   // [column][row], swizzled
    __shared__ float red[32];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int n0 = lane & 15, lg = lane >> 4;
    const int cp = t >> 2, pp = t & 3;     // column phase: column cp of the half, rows 64pp + [0, 64)
    const int64_t nct = a.cols / BT;
    const int64_t items = both_items(a.rows, a.cols);
    float s1 = 0.0f, r1 = 0.0f, sc2 = 0.0f, r2 = 0.0f;
    if constexpr (quant_op(OP)) {
      // the fallback pass after the single-pass kernel: nothing to do unless it aborted
      if (a.bar != nullptr && __hip_atomic_load(&a.bar[kReleaseWord], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) != kStateAborted)
        return;
      tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, s1, r1);
      tensor_scale(a.part_in2, a.nparts, a.step2, a.qmaxf, red, sc2, r2);
      zero_side(a);
      if (blockIdx.x == 0 && t == 0) {
        *a.scale_out = s1;
        *a.scale_out2 = sc2;
      }
    }
    const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
    constexpr int KM = K < 64 ? K : 64;
    constexpr int NKS = K > 128 ? 8 : 4;    // 32-column slices read per row block
    constexpr int NNB = K > 128 ? 16 : 8;   // 16-column output blocks computed
    uint4 G[4];
    hfrags<In, KM>(lane, G);
    const char* src = static_cast<const char*>(a.src);
    float amax1 = 0.0f, amax2 = 0.0f;
    const int64_t full = items / 16 * 16;
    auto decode = [&](int64_t it, int64_t& row0, int64_t& col0, int& h) {
      int64_t tl;
      if (it < full) {
        tl = (it / 16) * 8 + (it % 8);
        h = static_cast<int>((it / 8) & 1);
      } else {
        tl = full / 2 + (it - full) / 2;
        h = static_cast<int>((it - full) & 1);
      }
      row0 = (tl / nct) * BT;
      col0 = (tl % nct) * BT;
    };
    constexpr int RAWB = 2 * 32 * NKS;      // bytes of one raw row in LDS (512 or 256)
    constexpr int NCH = RAWB / 16, RPK = 1024 / RAWB;
    int8_t* const raw = reinterpret_cast<int8_t*>(half);
    // direct-to-LDS loads of item it's raw rows: 1 KB blocks w + 8i, lane l -> row
    // RPK (w + 8i) + l / NCH, slot l % NCH = chunk (l % NCH) ^ (row % 16)
    auto issue_raw = [&](int64_t it) {
      int64_t row0, col0;
      int h;
      decode(it, row0, col0, h);
      const int64_t ccol = col0 + (NKS == 8 ? 0 : BT_HALF * h);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(src + (row0 * a.cols + ccol) * 2), 0, static_cast<int>(BT * a.cols * 2),
          kBufferFlags);
#pragma unroll
      for (int i = 0; i < BT / RPK / 8; ++i) {
        const int b = w + 8 * i, r = RPK * b + lane / NCH, c = (lane % NCH) ^ (r & 15);
        lds_dma16(rs, raw + b * 1024, r * static_cast<int>(a.cols) * 2 + 16 * c);
      }
    };
    if constexpr (PIPE) {
      if (static_cast<int64_t>(blockIdx.x) < items) issue_raw(blockIdx.x);
    }
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
      int64_t row0, col0;
      int h;
      decode(it, row0, col0, h);
      const int64_t ccol = col0 + (NKS == 8 ? 0 : BT_HALF * h);   // first column read
      uint4 xr[PIPE ? 2 : 1][NKS];
      if constexpr (PIPE) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's raw loads landed
        __syncthreads();                                    // and every wave's
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int r = 32 * w + 16 * rb + n0;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            xr[rb][ks] = *reinterpret_cast<const uint4*>(raw + r * RAWB + 16 * ((4 * ks + lg) ^ (r & 15)));
        }
      }
      __syncthreads();   // the half tile is free: raw rows read, or the previous column phase done
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int rloc = 32 * w + 16 * rb;   // first tile row of this block
        uint4 x[NKS];
        if constexpr (PIPE) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) x[ks] = xr[rb][ks];
        } else {
          const char* p = src + ((row0 + rloc + n0) * a.cols + ccol + 8 * lg) * 2;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) x[ks] = *reinterpret_cast<const uint4*>(p + 64 * ks);
        }
        f32x4 acc[NNB];
        mma_rows<In, KM, NKS, NNB>(x, G, acc);
        mma_high_stages<K, NNB, 128>(acc);
        f32x4 y[8];
        if constexpr (K > 128) {
          const float sg = h ? -1.0f : 1.0f;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) y[nb][j] = __builtin_fmaf(acc[nb + 8][j], sg, acc[nb][j]);
        } else {
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) y[nb] = acc[nb];
        }
        if constexpr (OP == OP_ABSMAX) {
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) amax1 = fmaxf(amax1, fabsf(y[nb][j]));
        } else if (a.codes) {
          // After the byte transpose, lane (n0 = 4m + i, lg) holds the codes of columns
          // 16nb + 4m + [0, 4) of row 4lg + i; the dword transpose over m then gives lane m all
          // 16 codes of blocks m and 4 + m, two 16-byte stores (code rows are 16-byte aligned).
          // One store instruction covers 64 consecutive bytes of 16 rows: 4-byte stores covering
          // 16 bytes of each row wrote at about half the rate of whole lines.
          const int i = n0 & 3, m = n0 >> 2;
          uint32_t d[8];
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            d[nb] = quad_byte_transpose(
                quant4(y[nb][0], y[nb][1], y[nb][2], y[nb][3], r1, lo, hi, (OP == OP_QUANT_F8)), i);
          lane4_transpose(d[0], d[1], d[2], d[3]);
          lane4_transpose(d[4], d[5], d[6], d[7]);
          int8_t* dst = a.codes + (row0 + rloc + 4 * lg + i) * a.ld + col0 + BT_HALF * h + 16 * m;
          *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
          *reinterpret_cast<uint4*>(dst + 64) = make_uint4(d[4], d[5], d[6], d[7]);
        }
        const int c4 = (rloc >> 2) + lg;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int c = 16 * nb + n0;
          *reinterpret_cast<float4*>(&half[c * BT + 4 * bm_chunk(c, c4)]) =
              make_float4(y[nb][0], y[nb][1], y[nb][2], y[nb][3]);
        }
      }
      __syncthreads();
      // ---- column phase: the token-axis rotation of this half, in TokenT
      TokenT u[64];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 f = *reinterpret_cast<const float4*>(&half[cp * BT + 4 * bm_chunk(cp, 16 * pp + i)]);
        u[4 * i] = f.x;
        u[4 * i + 1] = f.y;
        u[4 * i + 2] = f.z;
        u[4 * i + 3] = f.w;
      }
      if constexpr (PIPE) {
        __syncthreads();   // every wave has its column values: the buffer takes the next raw rows
        if (it + gridDim.x < items) issue_raw(it + gridDim.x);
      }
      fwht_from<1, K, 64>(u);
      // strides 64 and 128 across the quad: fused DPP fmas, the upper lanes keeping negated
      // sums; the sign a lane collects goes into its reciprocal scale (exact)
      if constexpr (K > 64) xstage_signed<1>(u, (pp & 1) ? -1.0f : 1.0f);
      if constexpr (K > 128) xstage_signed<2>(u, (pp & 2) ? -1.0f : 1.0f);
      const float tsg = ((K > 64 && (pp & 1)) ? -1.0f : 1.0f) * ((K > 128 && (pp & 2)) ? -1.0f : 1.0f);
      const int64_t gcol = col0 + BT_HALF * h + cp;
      if constexpr (OP == OP_ABSMAX) {
#pragma unroll
        for (int i = 0; i < 64; ++i) amax2 = fmaxf(amax2, fabsf(static_cast<float>(u[i])));
      } else {
        // xq[q] holds rows 64pp + 16q + [0, 16) of the column. The quad's four lanes (pp) trade
        // those chunks, one dword index at a time, so that lane pp ends up with rows
        // 64q + 16pp + [0, 16): each store instruction then writes 64 consecutive bytes of a
        // column's code row instead of four 16-byte pieces 64 bytes apart, which wrote at about
        // half the rate of whole lines.
        uint32_t xq[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 16 * q + 4 * j;
            xq[q][j] = quant4(static_cast<float>(u[i]), static_cast<float>(u[i + 1]),
                              static_cast<float>(u[i + 2]), static_cast<float>(u[i + 3]),
                              r2 * tsg, lo, hi, (OP == OP_QUANT_F8));
          }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t col[4] = {xq[0][j], xq[1][j], xq[2][j], xq[3][j]};
          quad_transpose4(col, pp);
#pragma unroll
          for (int q = 0; q < 4; ++q) xq[q][j] = col[q];
        }
        int8_t* dst = a.codes_t + gcol * a.ld_t + row0 + 16 * pp;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint4*>(dst + 64 * q) = make_uint4(xq[q][0], xq[q][1], xq[q][2], xq[q][3]);
      }
    }
    if constexpr (OP == OP_ABSMAX) {
      amax1 = block_max(amax1, red);
      amax2 = block_max(amax2, red);
      if (t == 0) {
        a.partials[blockIdx.x] = amax1;
        a.partials[gridDim.x + blockIdx.x] = amax2;
      }
    }
  }
}

template <class In, int K, int OP>
__global__ __launch_bounds__(BM_THREADS) void both_mma_kernel(ProArgs a) {
  if constexpr (In::bytes == 2 && K >= 16) both_mma_body<In, K, OP, false>(a);
}

template <class In, int K, int OP>
__global__ __launch_bounds__(BM_THREADS) void both_pipe_kernel(ProArgs a) {
  if constexpr (In::bytes == 2 && K >= 16) both_mma_body<In, K, OP, true>(a);
}

// ================================================================ both, narrow items (k <= 128)
// With k <= 128 a token-axis block spans at most 128 rows and a feature-axis block at most 128
// columns, so a work item can be a 128 x 128 tile: its fp32 staging takes 64 KB of LDS instead of
// the 128 KB of a 256-row half tile, and two workgroups of four waves share a CU. Their load,
// matrix-core, LDS and butterfly phases then overlap, where a single 8-wave workgroup ran them
// in series. Per item, as both_pipe_kernel:
//  - the raw 16-bit rows (128 x 256 bytes) come in by direct-to-LDS loads issued during the
//    previous item's token phase, chunk c of row r at c ^ (r % 16);
//  - row phase on the matrix cores (wave w: rows 32w + [0, 32)), row-major codes of X B stored
//    from registers;
//  - X B staged column-major as fp32, 16-byte row chunk c4 of column c at
//    c4 ^ (c % 16) ^ 8 (c4 / 16): the 16-lane write groups (one chunk, 16 columns) and the read
//    groups (8 columns x both row halves) meet 16 distinct 16-byte bank groups;
//  - token phase: thread (column t / 2, half t % 2) rotates rows 64 (t % 2) + [0, 64) in fp32
//    registers, the stride-64 stage (k = 128) between the two lanes of a pair;
//  - transposed codes of B X B go through a 16 KB byte tile in the upper half of the staging
//    buffer (the raw rows of the next item use the lower half), column c's 16-byte chunk q at
//    q ^ ((c / 2) % 4), and leave as 16-byte stores of whole 128-byte column runs.
constexpr int BN_ROWS = 128, BN_COLS = 128, BN_THREADS = 256, BN_GRID = 512;

__host__ __device__ inline int64_t both_narrow_items(int64_t rows, int64_t cols) {
  return (rows / BN_ROWS) * (cols / BN_COLS);
}

// The narrow kernel takes the shapes of both_pipe_kernel (several items per workgroup) when
// k <= 128.
__host__ __device__ inline bool both_narrow_ok(int64_t rows, int64_t cols, bool vec, int in_bytes,
                                               int k) {
  return both_mma_ok(rows, cols, vec, in_bytes, k) && k <= BN_COLS &&
         both_items(rows, cols) > 256;
}

__device__ inline int bn_chunk(int c, int c4) { return c4 ^ (c & 15) ^ (8 * ((c4 >> 4) & 1)); }

template <class In, int K, int OP>
__global__ __launch_bounds__(BN_THREADS, 2) void both_narrow_kernel(ProArgs a) {
  if constexpr (In::bytes != 2 || K < 16 || K > BN_COLS) {
    return;
  } else {
    __shared__ __attribute__((aligned(16))) float half[BN_COLS * BN_ROWS];   // [column][row]
    __shared__ float red[32];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int n0 = lane & 15, lg = lane >> 4;
    const int cp = t >> 1, pp = t & 1;   // token phase: column cp, rows 64pp + [0, 64)
    const int64_t nct = a.cols / BN_COLS;
    const int64_t items = both_narrow_items(a.rows, a.cols);
    float s1 = 0.0f, r1 = 0.0f, sc2 = 0.0f, r2 = 0.0f;
    if constexpr (quant_op(OP)) {
      tensor_scale(a.part_in, a.nparts, a.step, a.qmaxf, red, s1, r1);
      tensor_scale(a.part_in2, a.nparts, a.step2, a.qmaxf, red, sc2, r2);
      zero_side(a);
      if (blockIdx.x == 0 && t == 0) {
        *a.scale_out = s1;
        *a.scale_out2 = sc2;
      }
    }
    const float lo = code_lo<OP>(a), hi = code_hi<OP>(a);
    constexpr int KM = K < 64 ? K : 64;
    constexpr int NKS = 4, NNB = 8;         // 32-column slices, 16-column output blocks
    constexpr int RAWB = 2 * BN_COLS;       // bytes of one raw row (256)
    constexpr int NCH = RAWB / 16, RPK = 1024 / RAWB;
    uint4 G[4];
    hfrags<In, KM>(lane, G);
    const char* src = static_cast<const char*>(a.src);
    int8_t* const raw = reinterpret_cast<int8_t*>(half);                 // bytes [0, 32 KB)
    uint4* const ctile = reinterpret_cast<uint4*>(half) + 2048;           // bytes [32, 48 KB)
    float amax1 = 0.0f, amax2 = 0.0f;
    // direct-to-LDS loads of item it's raw rows: 1 KB blocks w + 4i, lane l -> row
    // RPK (w + 4i) + l / NCH, slot l % NCH = chunk (l % NCH) ^ (row % 16)
    auto issue_raw = [&](int64_t it) {
      const int64_t ip = a.rev ? items - 1 - it : it;
      const int64_t row0 = (ip / nct) * BN_ROWS, col0 = (ip % nct) * BN_COLS;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(src + (row0 * a.cols + col0) * 2), 0,
          static_cast<int>(BN_ROWS * a.cols * 2), kBufferFlags);
#pragma unroll
      for (int i = 0; i < BN_ROWS / RPK / 4; ++i) {
        const int b = w + 4 * i, r = RPK * b + lane / NCH, c = (lane % NCH) ^ (r & 15);
        lds_dma16(rs, raw + b * 1024, r * static_cast<int>(a.cols) * 2 + 16 * c);
      }
    };
    if (static_cast<int64_t>(blockIdx.x) < items) issue_raw(blockIdx.x);
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
      const int64_t ip = a.rev ? items - 1 - it : it;
      const int64_t row0 = (ip / nct) * BN_ROWS, col0 = (ip % nct) * BN_COLS;
      uint4 xr[2][NKS];
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's raw loads landed
      __syncthreads();                                    // and every wave's
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * w + 16 * rb + n0;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          xr[rb][ks] = *reinterpret_cast<const uint4*>(raw + r * RAWB + 16 * ((4 * ks + lg) ^ (r & 15)));
      }
      __syncthreads();   // raw rows read by every wave: the buffer takes the fp32 tile
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int rloc = 32 * w + 16 * rb;   // first tile row of this block
        f32x4 y[NNB];
        mma_rows<In, KM, NKS, NNB>(xr[rb], G, y);
        mma_high_stages<K, NNB, 128>(y);
        if constexpr (OP == OP_ABSMAX) {
#pragma unroll
          for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) amax1 = fmaxf(amax1, fabsf(y[nb][j]));
        } else if (a.codes) {
          // as both_mma_body: after the byte and dword transposes lane (n0 = 4m + i, lg) holds
          // all 16 codes of column blocks m and 4 + m of row 4lg + i
          const int i = n0 & 3, m = n0 >> 2;
          uint32_t d[8];
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            d[nb] = quad_byte_transpose(
                quant4(y[nb][0], y[nb][1], y[nb][2], y[nb][3], r1, lo, hi, (OP == OP_QUANT_F8)), i);
          lane4_transpose(d[0], d[1], d[2], d[3]);
          lane4_transpose(d[4], d[5], d[6], d[7]);
          int8_t* dst = a.codes + (row0 + rloc + 4 * lg + i) * a.ld + col0 + 16 * m;
          *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
          *reinterpret_cast<uint4*>(dst + 64) = make_uint4(d[4], d[5], d[6], d[7]);
        }
        const int c4 = (rloc >> 2) + lg;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
          const int c = 16 * nb + n0;
          *reinterpret_cast<float4*>(&half[c * BN_ROWS + 4 * bn_chunk(c, c4)]) =
              make_float4(y[nb][0], y[nb][1], y[nb][2], y[nb][3]);
        }
      }
      __syncthreads();
      // ---- token phase
      float u[64];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 f = *reinterpret_cast<const float4*>(&half[cp * BN_ROWS + 4 * bn_chunk(cp, 16 * pp + i)]);
        u[4 * i] = f.x;
        u[4 * i + 1] = f.y;
        u[4 * i + 2] = f.z;
        u[4 * i + 3] = f.w;
      }
      __syncthreads();   // every wave has its column values: the lower half takes the next raw rows
      if (it + gridDim.x < items) issue_raw(it + gridDim.x);
      fwht_from<1, K, 64>(u);
      // stride 64 (k = 128): one fused DPP fma per value; the upper lane of each pair (pp = 1)
      // keeps the negated sums, so its quantizer takes the negated reciprocal (an exact sign)
      const float tsg = (K > 64 && pp) ? -1.0f : 1.0f;
      if constexpr (K > 64) xstage_signed<1>(u, tsg);
      if constexpr (OP == OP_ABSMAX) {
#pragma unroll
        for (int i = 0; i < 64; ++i) amax2 = fmaxf(amax2, fabsf(u[i]));
      } else {
        const float r2s = r2 * tsg;
        // rows 64pp + 16q + [0, 16) of column cp -> chunk 4pp + q of the column's 128-byte run
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 16 * q + 4 * j;
            d[j] = quant4(u[i], u[i + 1], u[i + 2], u[i + 3], r2s, lo, hi, (OP == OP_QUANT_F8));
          }
          ctile[8 * cp + ((4 * pp + q) ^ ((cp >> 1) & 3))] = make_uint4(d[0], d[1], d[2], d[3]);
        }
        __syncthreads();
        // eight lanes per column: store s covers columns 32s + t / 8, chunk t % 8 of each
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c = 32 * s + (t >> 3), ch = t & 7;
          const uint4 v = ctile[8 * c + (ch ^ ((c >> 1) & 3))];
          *reinterpret_cast<uint4*>(a.codes_t + (col0 + c) * a.ld_t + row0 + 16 * ch) = v;
        }
      }
    }
    if constexpr (OP == OP_ABSMAX) {
      amax1 = block_max(amax1, red);
      amax2 = block_max(amax2, red);
      if (t == 0) {
        a.partials[blockIdx.x] = amax1;
        a.partials[gridDim.x + blockIdx.x] = amax2;
      }
    }
  }
}

// ================================================================ both, single pass
// X under HALO-2 in ABSMAX mode when every workgroup has exactly one item (2048 x 4096 and
// smaller): the two passes in one launch. Each workgroup computes X B (kept in LDS, column-major
// as in both_mma) and B X B (kept in registers as fp32), publishes its two partial maxima with
// device-coherent stores, and arrives at a grid barrier: per-group arrival counters (eight
// groups), then a group-completion counter whose last arrival moves the state word from open to
// released with a compare-and-swap. Relaxed atomics only, so no cache-wide writeback is needed:
// the only data crossing workgroups are the partials, written and read at device scope. The
// others wait for the release a bounded time (a.spin polls), then read all partials, form both
// scales exactly as the two-pass kernels do, and write the codes of X B and B X B from what they
// kept. A workgroup whose wait runs out (some workgroup of the grid is not running yet) moves
// the state to aborted (unless it was released meanwhile) and leaves without writing codes;
// after an abort nobody writes codes, and the both_mma QUANT pass launched next on the stream
// (given a.bar) recomputes them all from the partials, which every workgroup publishes before
// it waits. Without an abort that pass returns at once. No wait is unbounded. The barrier words
// are zeroed by the launch before on the stream.
// One item of the single-pass kernel: compute() puts X B of the item in the LDS half tile (and
// returns this thread's maxima) and B X B of this thread's column segment in v2; emit() writes
// the item's codes from those with the given reciprocal scales.
template <class In, int K, bool F8>
struct BothItem {
  static constexpr int KM = K < 64 ? K : 64, NKS = K > 128 ? 8 : 4, NNB = K > 128 ? 16 : 8;
  const ProArgs& a;
  float* half;
  int t, lane, w, n0, lg, cp, pp;
  int64_t nct, items, full;
  uint4 G[4];
  float v2[64];
  __device__ BothItem(const ProArgs& args, float* h) : a(args), half(h) {
    t = threadIdx.x;
    lane = t & 63;
    w = t >> 6;
    n0 = lane & 15;
    lg = lane >> 4;
    cp = t >> 2;
    pp = t & 3;
    nct = a.cols / BT;
    items = both_items(a.rows, a.cols);
    full = items / 16 * 16;
    hfrags<In, KM>(lane, G);
  }
  __device__ void decode(int64_t it, int64_t& row0, int64_t& col0, int& h) const {
    int64_t tl;
    if (it < full) {
      tl = (it / 16) * 8 + (it % 8);
      h = static_cast<int>((it / 8) & 1);
    } else {
      tl = full / 2 + (it - full) / 2;
      h = static_cast<int>((it - full) & 1);
    }
    row0 = (tl / nct) * BT;
    col0 = (tl % nct) * BT;
  }
  __device__ void compute(int64_t it, float& m1, float& m2) {
    int64_t row0, col0;
    int h;
    decode(it, row0, col0, h);
    const int64_t ccol = col0 + (NKS == 8 ? 0 : BT_HALF * h);
    const char* src = static_cast<const char*>(a.src);
    __syncthreads();   // the previous item's readers of the half tile are done
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int rloc = 32 * w + 16 * rb;
      const char* p = src + ((row0 + rloc + n0) * a.cols + ccol + 8 * lg) * 2;
      uint4 x[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) x[ks] = *reinterpret_cast<const uint4*>(p + 64 * ks);
      f32x4 acc[NNB];
      mma_rows<In, KM, NKS, NNB>(x, G, acc);
      mma_high_stages<K, NNB, 128>(acc);
      f32x4 y[8];
      if constexpr (K > 128) {
        const float sg = h ? -1.0f : 1.0f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) y[nb][j] = __builtin_fmaf(acc[nb + 8][j], sg, acc[nb][j]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) y[nb] = acc[nb];
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) m1 = fmaxf(m1, fabsf(y[nb][j]));
      const int c4 = (rloc >> 2) + lg;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int c = 16 * nb + n0;
        *reinterpret_cast<float4*>(&half[c * BT + 4 * bm_chunk(c, c4)]) =
            make_float4(y[nb][0], y[nb][1], y[nb][2], y[nb][3]);
      }
    }
    __syncthreads();
    TokenT u[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 f = *reinterpret_cast<const float4*>(&half[cp * BT + 4 * bm_chunk(cp, 16 * pp + i)]);
      u[4 * i] = f.x;
      u[4 * i + 1] = f.y;
      u[4 * i + 2] = f.z;
      u[4 * i + 3] = f.w;
    }
    fwht_from<1, K, 64>(u);
    // fused DPP fmas, the upper lanes keeping negated sums (emit() folds the sign into r2)
    if constexpr (K > 64) xstage_signed<1>(u, (pp & 1) ? -1.0f : 1.0f);
    if constexpr (K > 128) xstage_signed<2>(u, (pp & 2) ? -1.0f : 1.0f);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      v2[i] = static_cast<float>(u[i]);
      m2 = fmaxf(m2, fabsf(v2[i]));
    }
  }
  // Codes of the item: quantized into registers, then staged back through the half-tile
  // buffer (its fp32 values are no longer needed) so that both layouts leave as 16-byte stores
  // covering whole lines: the row-major X B codes as a 256 x 128-byte tile (dword d of row r
  // at d ^ 4((r / 2) % 8): the accumulator-layout writes meet 64 distinct banks), the B X B
  // codes_t as a 128 x 256-byte tile (16-byte chunk k of row r at k ^ (r % 16)).
  __device__ void emit(int64_t it, float r1, float r2) const {
    int64_t row0, col0;
    int h;
    decode(it, row0, col0, h);
    const float lo = code_lo<F8 ? OP_QUANT_F8 : OP_QUANT>(a), hi = code_hi<F8 ? OP_QUANT_F8 : OP_QUANT>(a);
    const int i = n0 & 3, m = n0 >> 2;
    uint32_t rc[2][8];
    if (a.codes) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int c4 = ((32 * w + 16 * rb) >> 2) + lg;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int c = 16 * nb + n0;
          const float4 y = *reinterpret_cast<const float4*>(&half[c * BT + 4 * bm_chunk(c, c4)]);
          const uint32_t d = quant4(y.x, y.y, y.z, y.w, r1, lo, hi, F8);
          rc[rb][nb] = quad_byte_transpose(d, i);
        }
      }
    }
    uint32_t tc[16];
    const float r2s = r2 * ((K > 64 && (pp & 1)) ? -1.0f : 1.0f) * ((K > 128 && (pp & 2)) ? -1.0f : 1.0f);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      tc[j] = quant4(v2[4 * j], v2[4 * j + 1], v2[4 * j + 2], v2[4 * j + 3], r2s, lo, hi, F8);
    __syncthreads();   // every thread has read its values out of the half tile
    uint32_t* const rt = reinterpret_cast<uint32_t*>(half);   // [256 rows][32 dwords]
    uint32_t* const ct = rt + 256 * 32;                       // [128 columns][64 dwords]
    if (a.codes) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = 32 * w + 16 * rb + 4 * lg + i;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) rt[row * 32 + ((4 * nb + m) ^ (4 * ((row >> 1) & 7)))] = rc[rb][nb];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(&ct[cp * 64 + 4 * ((4 * pp + q) ^ (cp & 15))]) =
          make_uint4(tc[4 * q], tc[4 * q + 1], tc[4 * q + 2], tc[4 * q + 3]);
    __syncthreads();
    if (a.codes) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int idx = BM_THREADS * p + t, row = idx >> 3, c = idx & 7;
        *reinterpret_cast<uint4*>(a.codes + (row0 + row) * a.ld + col0 + BT_HALF * h + 16 * c) =
            *reinterpret_cast<const uint4*>(&rt[row * 32 + 4 * (c ^ ((row >> 1) & 7))]);
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = BM_THREADS * p + t, rr = idx >> 4, k = idx & 15;
      *reinterpret_cast<uint4*>(a.codes_t + (col0 + BT_HALF * h + rr) * a.ld_t + row0 + 16 * k) =
          *reinterpret_cast<const uint4*>(&ct[rr * 64 + 4 * (k ^ (rr & 15))]);
    }
  }
};

template <class In, int K, bool F8>
__global__ __launch_bounds__(BM_THREADS) void both_single_kernel(ProArgs a) {
  if constexpr (In::bytes != 2 || K < 16) {
    return;
  } else {
    __shared__ __attribute__((aligned(16))) float half[BT_HALF * BT];   // [column][row], swizzled
    __shared__ float red[32];
    __shared__ int s_state;
    constexpr int OPEN = 0, RELEASED = 1, ABORTED = 2;
    const int t = threadIdx.x, wg = blockIdx.x, nwg = gridDim.x;   // nwg == items (host checks)
    BothItem<In, K, F8> b(a, half);
    float amax1 = 0.0f, amax2 = 0.0f;
    b.compute(wg, amax1, amax2);
    // ---- partial maxima, grid barrier
    amax1 = block_max(amax1, red);
    amax2 = block_max(amax2, red);
    if (t == 0) {
      __hip_atomic_store(reinterpret_cast<int*>(a.partials) + wg, __float_as_int(amax1),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(reinterpret_cast<int*>(a.partials) + nwg + wg, __float_as_int(amax2),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      int* const state = &a.bar[kReleaseWord];
      const int grp = wg % kBarGroups, gsize = (nwg - grp + kBarGroups - 1) / kBarGroups;
      const int old = __hip_atomic_fetch_add(&a.bar[kBarStride * grp], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      bool last = false;
      if (old == gsize - 1)
        last = __hip_atomic_fetch_add(&a.bar[kGroupDone], 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == kBarGroups - 1;
      int st;
      if (last) {
        // release; a failed swap means some workgroup gave up: the fallback pass redoes it all
        int expect = OPEN;
        st = __hip_atomic_compare_exchange_strong(state, &expect, RELEASED, __ATOMIC_RELAXED,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 ? RELEASED
                 : ABORTED;
      } else {
        st = OPEN;
        for (int i = 0; i <= a.spin && st == OPEN; ++i) {
          st = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (st == OPEN && i < a.spin) __builtin_amdgcn_s_sleep(1);
        }
        if (st == OPEN) {
          int expect = OPEN;
          st = __hip_atomic_compare_exchange_strong(state, &expect, ABORTED, __ATOMIC_RELAXED,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   ? ABORTED
                   : expect;
        }
      }
      s_state = st;
    }
    __syncthreads();
    if (s_state != RELEASED) return;
    // ---- scales from every partial (as tensor_scale), then the codes
    float p1 = 0.0f, p2 = 0.0f;
    for (int i = t; i < nwg; i += BM_THREADS) {
      p1 = fmaxf(p1, __int_as_float(__hip_atomic_load(reinterpret_cast<int*>(a.partials) + i,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
      p2 = fmaxf(p2, __int_as_float(__hip_atomic_load(reinterpret_cast<int*>(a.partials) + nwg + i,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    }
    p1 = block_max(p1, red);
    p2 = block_max(p2, red);
    const float s1 = p1 / a.qmaxf, s2 = p2 / a.qmaxf;
    const float r1 = (s1 > 0.0f) ? 1.0f / s1 : 0.0f, r2 = (s2 > 0.0f) ? 1.0f / s2 : 0.0f;
    if (wg == 0 && t == 0) {
      *a.scale_out = s1;
      *a.scale_out2 = s2;
    }
    b.emit(wg, r1, r2);
  }
}

// ================================================================ launchers
static int grid_cap(int64_t tiles, int cap) {
  if (tiles < 1) tiles = 1;
  return static_cast<int>(tiles < cap ? tiles : cap);
}

template <template <class, int, int> class KERN, int OP>
struct Launch;

#define HQ_PRO_DISPATCH(NAME, THREADS)                                                         \
  template <class In, int OP>                                                                  \
  static hipError_t NAME##_k(int k, const ProArgs& a, int grid, hipStream_t st, int tok) {    \
    switch (k) {                                                                               \
      case 1: return launch_k(NAME<In, 1, OP>, dim3(grid), dim3(THREADS), st, tok, a);           \
      case 2: return launch_k(NAME<In, 2, OP>, dim3(grid), dim3(THREADS), st, tok, a);           \
      case 4: return launch_k(NAME<In, 4, OP>, dim3(grid), dim3(THREADS), st, tok, a);           \
      case 8: return launch_k(NAME<In, 8, OP>, dim3(grid), dim3(THREADS), st, tok, a);           \
      case 16: return launch_k(NAME<In, 16, OP>, dim3(grid), dim3(THREADS), st, tok, a);         \
      case 32: return launch_k(NAME<In, 32, OP>, dim3(grid), dim3(THREADS), st, tok, a);         \
      case 64: return launch_k(NAME<In, 64, OP>, dim3(grid), dim3(THREADS), st, tok, a);         \
      case 128: return launch_k(NAME<In, 128, OP>, dim3(grid), dim3(THREADS), st, tok, a);       \
      case 256: return launch_k(NAME<In, 256, OP>, dim3(grid), dim3(THREADS), st, tok, a);       \
      default: return hipErrorInvalidValue;                                                    \
    }                                                                                          \
  }                                                                                            \
  static hipError_t NAME##_launch(int in_dt, int op, int k, const ProArgs& a, int grid,        \
                                  hipStream_t st, int tok) {                                   \
    if (op == OP_ABSMAX) {                                                                     \
      switch (in_dt) {                                                                         \
        case DT_F32: return NAME##_k<F32, OP_ABSMAX>(k, a, grid, st, tok);                          \
        case DT_F16: return NAME##_k<F16, OP_ABSMAX>(k, a, grid, st, tok);                          \
        case DT_BF16: return NAME##_k<BF16, OP_ABSMAX>(k, a, grid, st, tok);                        \
      }                                                                                        \
    } else if (op == OP_QUANT) {                                                               \
      switch (in_dt) {                                                                         \
        case DT_F32: return NAME##_k<F32, OP_QUANT>(k, a, grid, st, tok);                           \
        case DT_F16: return NAME##_k<F16, OP_QUANT>(k, a, grid, st, tok);                           \
        case DT_BF16: return NAME##_k<BF16, OP_QUANT>(k, a, grid, st, tok);                         \
      }                                                                                        \
    } else if (op == OP_QUANT_F8) {                                                            \
      switch (in_dt) {                                                                         \
        case DT_F32: return NAME##_k<F32, OP_QUANT_F8>(k, a, grid, st, tok);                        \
        case DT_F16: return NAME##_k<F16, OP_QUANT_F8>(k, a, grid, st, tok);                        \
        case DT_BF16: return NAME##_k<BF16, OP_QUANT_F8>(k, a, grid, st, tok);                      \
      }                                                                                        \
    }                                                                                          \
    return hipErrorInvalidValue;                                                               \
  }

HQ_PRO_DISPATCH(right_kernel, RT_THREADS)
HQ_PRO_DISPATCH(right_fast_kernel, RF_THREADS)
HQ_PRO_DISPATCH(right_mma_kernel, RM_THREADS)
HQ_PRO_DISPATCH(left_kernel, LT_THREADS)
HQ_PRO_DISPATCH(left_fast_kernel, LF_THREADS)
HQ_PRO_DISPATCH(left_mma_kernel, LM_THREADS)
HQ_PRO_DISPATCH(both_kernel, BT_THREADS)
HQ_PRO_DISPATCH(both_mma_kernel, BM_THREADS)
HQ_PRO_DISPATCH(both_pipe_kernel, BM_THREADS)
#undef HQ_PRO_DISPATCH

template <class In, int OP>
static hipError_t both_narrow_k(int k, const ProArgs& a, int grid, hipStream_t st, int tok) {
  switch (k) {
#define HQ_BN(KK) \
  case KK: return launch_k(both_narrow_kernel<In, KK, OP>, dim3(grid), dim3(BN_THREADS), st, tok, a);
    HQ_BN(16) HQ_BN(32) HQ_BN(64) HQ_BN(128)
#undef HQ_BN
  }
  return hipErrorInvalidValue;
}

template <class In>
static hipError_t both_narrow_op(int op, int k, const ProArgs& a, int grid, hipStream_t st, int tok) {
  if (op == OP_ABSMAX) return both_narrow_k<In, OP_ABSMAX>(k, a, grid, st, tok);
  if (op == OP_QUANT) return both_narrow_k<In, OP_QUANT>(k, a, grid, st, tok);
  if (op == OP_QUANT_F8) return both_narrow_k<In, OP_QUANT_F8>(k, a, grid, st, tok);
  return hipErrorInvalidValue;
}

static hipError_t both_narrow_launch(int in_dt, int op, int k, const ProArgs& a, int grid,
                                     hipStream_t st, int tok) {
  if (in_dt == DT_F16) return both_narrow_op<F16>(op, k, a, grid, st, tok);
  if (in_dt == DT_BF16) return both_narrow_op<BF16>(op, k, a, grid, st, tok);
  return hipErrorInvalidValue;
}

template <class In, bool F8>
static hipError_t both_single_k(int k, const ProArgs& a, int grid, hipStream_t st, int tok) {
  switch (k) {
#define HQ_BS(KK) \
  case KK: return launch_k(both_single_kernel<In, KK, F8>, dim3(grid), dim3(BM_THREADS), st, tok, a);
    HQ_BS(16) HQ_BS(32) HQ_BS(64) HQ_BS(128) HQ_BS(256)
#undef HQ_BS
  }
  return hipErrorInvalidValue;
}

static int dtb(int dt) { return dt == DT_F32 ? 4 : 2; }

// The narrow two-sided kernel is the default where it applies; HQ_BOTH_NARROW=0 selects
// both_pipe_kernel instead (read on every call, so a test can compare the two).
static bool both_narrow_on() {
  const char* e = std::getenv("HQ_BOTH_NARROW");
  return !(e && e[0] == '0');
}

static bool quant_reverse_on() {
  const char* e = std::getenv("HQ_QUANT_REVERSE");
  return !(e && e[0] == '0');
}

// The matrix-core kernels are the default for the shapes they take; HQ_PROLOGUE_VALU=1 runs
// every prologue pass on the VALU butterfly kernels instead, to measure one against the other.
static bool prologue_mma_on() {
  const char* e = std::getenv("HQ_PROLOGUE_VALU");
  return !(e && e[0] == '1');
}

static ProArgs pro_args(const ProPass& p) {
  ProArgs a{};
  a.src = p.src;
  a.rows = p.rows;
  a.cols = p.cols;
  a.vec = (reinterpret_cast<uintptr_t>(p.src) & 15u) == 0 && (p.cols * dtb(p.in_dt)) % 16 == 0;
  a.partials = p.partials;
  a.part_in = p.partials;
  a.part_in2 = p.partials + p.nparts;
  a.nparts = p.nparts;
  a.step = p.step;
  a.step2 = p.step2;
  a.qp = p.qp;
  a.qmaxf = p.qmaxf;
  a.fgrid = p.fgrid;
  a.scale_out = p.scale_out;
  a.scale_out2 = p.scale_out2;
  a.codes = p.codes;
  a.ld = p.ld;
  a.codes_t = p.codes_t;
  a.ld_t = p.ld_t;
  a.zero_ptr = p.zero_ptr;
  a.zero_n = p.zero_n;
  return a;
}

int pro_grid(const ProPass& p) {
  int64_t tiles;
  const bool mma = prologue_mma_on();
  if (p.kind == PRO_RIGHT) {
    if (mma && right_mma_ok(p.rows, p.cols, pro_args(p).vec, dtb(p.in_dt), p.k))
      return grid_cap((p.rows / RM_ROWS) * (p.cols / RM_COLS), RM_GRID);
    if (right_fast_ok(p.rows, p.cols, pro_args(p).vec))
      return grid_cap((p.rows / RF_ROWS) * (p.cols / RF_COLS), RF_GRID);
    tiles = ((p.rows + RT_ROWS - 1) / RT_ROWS) * ((p.cols + RT_COLS - 1) / RT_COLS);
  } else if (p.kind == PRO_LEFT) {
    if (mma && left_mma_ok(p.rows, p.cols, pro_args(p).vec, dtb(p.in_dt), p.k))
      return grid_cap((p.rows / LM_ROWS) * (p.cols / LM_COLS), LM_GRID);
    if (left_fast_ok(p.rows, p.cols, pro_args(p).vec, dtb(p.in_dt)))
      return grid_cap((p.rows / LF_ROWS) * (p.cols / LF_COLS), LF_GRID);
    const int tr = p.k > 64 ? p.k : 64, tc = LT_ELEMS / tr;
    tiles = ((p.rows + tr - 1) / tr) * ((p.cols + tc - 1) / tc);
  } else {
    if (mma && both_narrow_on() && both_narrow_ok(p.rows, p.cols, pro_args(p).vec, dtb(p.in_dt), p.k))
      return grid_cap(both_narrow_items(p.rows, p.cols), BN_GRID);   // two per CU
    // one 135 KB workgroup per CU: at most one item per CU at a time
    return grid_cap(both_items(p.rows, p.cols), 256);
  }
  return grid_cap(tiles, kMaxPartials);
}

hipError_t pro_pass(const ProPass& p, int op, hipStream_t st) {
  if (op == OP_QUANT && p.f8) op = OP_QUANT_F8;   // the quantize pass writing E4M3 codes
  ProArgs a = pro_args(p);
  // After an absmax pass over an input of 128 MiB or more (half the 256 MB memory-side cache)
  // the quantize pass visits the tiles in the opposite order, so it starts on the part read
  // last, which the cache still holds. Measured at 8192 x 13824 x 5120: W's pass (141.6 MB)
  // 62.3 -> 53.6 us, X's (226.5 MB) 94.4 -> 90.8 us; for the 84-90 MB tensors the reversed
  // order was 0.8 us slower, so they keep the forward order. HQ_QUANT_REVERSE=0 never reverses.
  a.rev = quant_op(op) && p.step == nullptr && quant_reverse_on() &&
          static_cast<double>(p.rows) * p.cols * dtb(p.in_dt) >= 134217728.0;
  const int grid = pro_grid(p);
  const double elems = static_cast<double>(p.rows) * p.cols;
  const double inb = elems * dtb(p.in_dt);
  double outb = 0.0;
  if (quant_op(op)) outb = elems * ((p.codes ? 1 : 0) + (p.codes_t ? 1 : 0));
  const int tok = prof_open(op == OP_ABSMAX ? K_ROT_ABSMAX : K_ROT_QUANT, inb + outb);
  hipError_t e = hipErrorInvalidValue;
  const bool mma = prologue_mma_on();
  if (p.kind == PRO_RIGHT && mma && right_mma_ok(p.rows, p.cols, a.vec, dtb(p.in_dt), p.k))
    e = right_mma_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (p.kind == PRO_RIGHT && right_fast_ok(p.rows, p.cols, a.vec))
    e = right_fast_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (p.kind == PRO_RIGHT) e = right_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (p.kind == PRO_LEFT && mma && left_mma_ok(p.rows, p.cols, a.vec, dtb(p.in_dt), p.k))
    e = left_mma_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (p.kind == PRO_LEFT && left_fast_ok(p.rows, p.cols, a.vec, dtb(p.in_dt)))
    e = left_fast_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (p.kind == PRO_LEFT) e = left_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (mma && both_narrow_on() && both_narrow_ok(p.rows, p.cols, a.vec, dtb(p.in_dt), p.k))
    e = both_narrow_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (mma && both_mma_ok(p.rows, p.cols, a.vec, dtb(p.in_dt), p.k) &&
           both_items(p.rows, p.cols) > grid)
    e = both_pipe_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else if (mma && both_mma_ok(p.rows, p.cols, a.vec, dtb(p.in_dt), p.k))
    e = both_mma_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  else e = both_kernel_launch(p.in_dt, op, p.k, a, grid, st, tok);
  return e;
}

// The matrix-core store mode covers whole 64 x 256 tiles of 16-bit data for every k >= 16. The
// automatic choice does not take it for RIGHT: with DPP lane exchanges the VALU rows kernel
// streams at least as fast at every k (measured on bf16 8192 x 13824).
bool fwht_right_mma_ok(const void* src, int dt, const void* dst, int out_dt, int64_t rows,
                       int64_t cols, int k) {
  const bool al = (reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                  (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  return dt == out_dt && (dt == DT_F16 || dt == DT_BF16) && al &&
         right_mma_ok(rows, cols, (cols * 2) % 16 == 0, 2, k);
}

hipError_t fwht_right_mma(const void* src, int dt, int64_t rows, int64_t cols, int k, void* dst,
                          hipStream_t st) {
  ProArgs a{};
  a.src = src;
  a.rows = rows;
  a.cols = cols;
  a.vec = true;
  a.dst = dst;
  const int grid = grid_cap((rows / RM_ROWS) * (cols / RM_COLS), RM_GRID);
  const int tok = prof_open(K_ROT_STORE, 4.0 * static_cast<double>(rows) * cols);
  return dt == DT_F16 ? right_mma_kernel_k<F16, OP_STORE>(k, a, grid, st, tok)
                      : right_mma_kernel_k<BF16, OP_STORE>(k, a, grid, st, tok);
}

bool fwht_left_mma_ok(const void* src, int dt, const void* dst, int out_dt, int64_t rows,
                      int64_t cols, int k) {
  const bool al = (reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                  (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  return dt == out_dt && (dt == DT_F16 || dt == DT_BF16) && al &&
         left_mma_ok(rows, cols, (cols * 2) % 16 == 0, 2, k);
}

hipError_t fwht_left_mma(const void* src, int dt, int64_t rows, int64_t cols, int k, void* dst,
                         hipStream_t st) {
  ProArgs a{};
  a.src = src;
  a.rows = rows;
  a.cols = cols;
  a.vec = true;
  a.dst = dst;
  const int grid = grid_cap((rows / LM_ROWS) * (cols / LM_COLS), LM_GRID);
  const int tok = prof_open(K_ROT_STORE, 4.0 * static_cast<double>(rows) * cols);
  return dt == DT_F16 ? left_mma_kernel_k<F16, OP_STORE>(k, a, grid, st, tok)
                      : left_mma_kernel_k<BF16, OP_STORE>(k, a, grid, st, tok);
}

bool pro_single_ok(const ProPass& p, int cus) {
  const ProArgs a = pro_args(p);
  return p.kind == PRO_BOTH && p.step == nullptr && prologue_mma_on() &&
         both_mma_ok(p.rows, p.cols, a.vec, dtb(p.in_dt), p.k) &&
         both_items(p.rows, p.cols) <= std::min(256, cus);
}

hipError_t pro_single_pass(const ProPass& p, int32_t* bar, hipStream_t st) {
  ProArgs a = pro_args(p);
  a.bar = bar;
  a.spin = 40000;   // polls of ~30 ns: about 1 ms before the fallback takes over
  if (const char* e = std::getenv("HQ_SINGLE_SPIN")) a.spin = std::max(0, std::atoi(e));
  const int grid = static_cast<int>(both_items(p.rows, p.cols));
  const double elems = static_cast<double>(p.rows) * p.cols;
  const int tok = prof_open(K_ROT_ABSMAX, elems * (2.0 + (p.codes ? 1 : 0) + (p.codes_t ? 1 : 0)));
  if (p.f8)
    return p.in_dt == DT_F16 ? both_single_k<F16, true>(p.k, a, grid, st, tok)
                             : both_single_k<BF16, true>(p.k, a, grid, st, tok);
  return p.in_dt == DT_F16 ? both_single_k<F16, false>(p.k, a, grid, st, tok)
                           : both_single_k<BF16, false>(p.k, a, grid, st, tok);
}

hipError_t pro_fixup_pass(const ProPass& p, int32_t* bar, hipStream_t st) {
  ProArgs a = pro_args(p);
  a.bar = bar;
  const int grid = pro_grid(p);
  const double elems = static_cast<double>(p.rows) * p.cols;
  const int tok = prof_open(K_ROT_QUANT, elems * ((p.codes ? 1 : 0) + (p.codes_t ? 1 : 0)));
  return both_mma_kernel_launch(p.in_dt, p.f8 ? OP_QUANT_F8 : OP_QUANT, p.k, a, grid, st, tok);
}

}  // namespace hq
