// Q4_0 prefill GEMM: m tokens x Q4_0 weights on the fp32 matrix cores.
//
// Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html), sections 2 and 3:
// 18-byte blocks of 32 weights (fp16 scale d, then 16 bytes of nibbles, the
// low nibble the even element), weight = (nibble - 8) * d, rows zero-padded
// to whole blocks.  "14MB holds 45M parameters" (Needle article), section 3:
// prefill is a GEMM over the same [out, in] layout, every row one reduction
// stream.  The sum is the Q4_0 GEMV's for m tokens:
//   y[t, r] = sum_blk sum_{j<32} ((nib[r, blk, j] - 8) * d[r, blk]) * x[t, 32 blk + j]
// with x taken as 0 past `cols` (the padded weights there are 0 too).
//
// Design:
//  * v_mfma_f32_32x32x2_f32: A = 32 tokens x 2 k (fp32 activations as they
//    come), B = 2 k x 32 weight rows, the weight (nibble - 8) * d formed in
//    fp32, where it is exact (a 4-bit integer times an fp16 value).  Products
//    and sums are fp32; nothing is rounded to a narrower type.
//  * Within a block, lane half h (= lane / 32) supplies elements 16 h .. 16 h
//    + 15 over the block's 16 MFMA steps (step s: element 16 h + s).  So a
//    lane reads 64 contiguous bytes of its token's activations and bytes
//    8 h .. 8 h + 7 of its row's nibbles (nibbles 16 h .. 16 h + 15), and A
//    and B agree on the order.
//  * A 256-thread workgroup computes a 64-token x 64-row tile as 2 x 2 wave
//    tiles of 32 x 32; every wave loads its own operands (they are small and
//    cached) and has the next block's loads in flight while it multiplies.
//    Where such tiles leave CUs idle (the small layer matrices), a workgroup
//    takes one 32 x 32 tile instead and its four waves split the blocks
//    (wave w: blocks w, w + 4, ...); their sums meet in LDS in a fixed order.
//    An fp32 MFMA occupies a SIMD for 64 cycles, so the split is what shortens
//    a small launch.  Rows of at most 16 blocks take 16 x 16 tiles on
//    v_mfma_f32_16x16x4_f32 instead (q4_0_gemm16_kernel), split the same way.
//  * Blocks sit at 2-byte-aligned offsets: the nibble bytes come as the 12
//    bytes from the 4-byte-aligned address below them, realigned with
//    v_alignbyte; the scale as the aligned word holding it.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kGemmThreads = 256;
constexpr int kQBlock = 32;
constexpr int kQBlockBytes = 18;
constexpr int kTileM = 64, kTileN = 64;      // tokens x weight rows per workgroup
constexpr uint32_t kOOBq = 0x80000000u;      // buffer offset past every range: reads give 0
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4q __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3q __attribute__((ext_vector_type(3)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_q(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// One block's operands for a lane: 16 activations and the raw words holding
// the scale and the lane's 8 nibble bytes.
struct BlockIn {
  float a[16];
  u32x3q nib;        // 12 bytes from the aligned address below the nibble bytes
  uint32_t dw;       // the aligned word holding the fp16 scale
};

// VEC: cols % 4 == 0 (x 16-byte aligned), so a lane's activations come as
// four 16-byte loads; otherwise as sixteen 4-byte loads.  KSPLIT: 1 (2 x 2
// wave tiles) or 4 (one tile, blocks split over the waves).
template <bool VEC, int KSPLIT>
__global__ __launch_bounds__(kGemmThreads) void q4_0_gemm_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t block_bytes,
    const float *__restrict__ x, uint32_t x_bytes, int m, float *__restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  constexpr int TM = KSPLIT == 1 ? kTileM : 32, TN = KSPLIT == 1 ? kTileN : 32;
  const int wm = KSPLIT == 1 ? (wave & 1) : 0, wn = KSPLIT == 1 ? (wave >> 1) : 0;
  const int kw = KSPLIT == 1 ? 0 : wave;                           // first block of this wave
  const int tok = blockIdx.y * TM + 32 * wm + l32;                 // A row of this lane
  const int row = blockIdx.x * TN + 32 * wn + l32;                 // B column of this lane
  const __amdgpu_buffer_rsrc_t rx = rsrc_q(x, x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc_q(blocks, block_bytes);
  // activations of block b: x[tok, 32 b + 16 h ..] (out of range: zeros)
  const uint32_t xrow = tok < m ? (uint32_t)tok * (uint32_t)cols * 4u : kOOBq;
  const uint32_t wrow = row < rows ? (uint32_t)row * (uint32_t)nblk * kQBlockBytes : kOOBq;

  auto load = [&](BlockIn &in, int b) {
    const uint32_t xo = xrow + (uint32_t)(kQBlock * b + 16 * h) * 4u;
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (the whole vector is converted: a bit_cast of one vector element
        // reads the vector's first element with this compiler)
        const f32x4q v = __builtin_bit_cast(f32x4q, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16u * i, 0, 0));
        in.a[4 * i + 0] = v.x;
        in.a[4 * i + 1] = v.y;
        in.a[4 * i + 2] = v.z;
        in.a[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        in.a[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, xo + 4u * i, 0, 0));
    }
    const uint32_t bo = wrow + (uint32_t)b * kQBlockBytes;
    in.dw = __builtin_amdgcn_raw_buffer_load_b32(rw, bo & ~3u, 0, 0);
    in.nib = __builtin_bit_cast(u32x3q, __builtin_amdgcn_raw_buffer_load_b96(rw, (bo + 2u + 8u * h) & ~3u, 0, 0));
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  auto multiply = [&](BlockIn &in, int b) {
    // activations past cols are taken as 0 (only the last block has any)
    if (b == nblk - 1 && (cols & (kQBlock - 1))) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (kQBlock * b + 16 * h + s >= cols) in.a[s] = 0.0f;
    }
    // the scale, and the lane's nibble bytes realigned (blocks are 2-byte aligned)
    const uint32_t bo = wrow + (uint32_t)b * kQBlockBytes;
    const float d = half_bits_to_float((uint16_t)(in.dw >> ((bo & 2u) * 8u)));
    const uint32_t sh = (bo + 2u + 8u * h) & 3u;
    uint32_t q[2];
    q[0] = __builtin_amdgcn_alignbyte(in.nib.y, in.nib.x, sh) ^ 0x88888888u;
    q[1] = __builtin_amdgcn_alignbyte(in.nib.z, in.nib.y, sh) ^ 0x88888888u;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      // element 16 h + s: nibble s of the 8 bytes, low nibble first; xor 8
      // and a signed 4-bit extract give nibble - 8
      const int v = __builtin_amdgcn_sbfe((int)q[s >> 3], 4 * (s & 7), 4);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(in.a[s], (float)v * d, acc, 0, 0, 0);
    }
  };
  // two buffers in turn: block b + 1's loads go out before block b is
  // multiplied (kept in place against the scheduler); loads past the last
  // block read block nblk - 1 again and are not used
  // the wave's blocks kw, kw + KSPLIT, ...; loads past its last block read
  // block nblk - 1 and are not used
  constexpr int S = KSPLIT;
  const int last = nblk - 1;
  BlockIn in0, in1;
  load(in0, kw < nblk ? kw : last);
  for (int b = kw; b < nblk; b += 2 * S) {
    load(in1, b + S < nblk ? b + S : last);
    __builtin_amdgcn_sched_barrier(0);
    multiply(in0, b);
    __builtin_amdgcn_sched_barrier(0);
    if (b + S < nblk) {                          // uniform
      load(in0, b + 2 * S < nblk ? b + 2 * S : last);
      __builtin_amdgcn_sched_barrier(0);
      multiply(in1, b + S);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (KSPLIT > 1) {
    // waves 1..3 hand their sums to wave 0, which adds them in wave order
    __shared__ float part[KSPLIT - 1][16][64];
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part[wave - 1][r][lane] = acc[r];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += part[w][r][lane];
  }

  // lane (l32, h) holds row l32 of the wave tile's columns and tokens
  // 8 i + 4 h + r (i, r < 4) of its rows
  if (row < rows) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = blockIdx.y * TM + 32 * wm + 8 * i + 4 * h + r;
        if (t < m) y[(size_t)t * rows + row] = acc[4 * i + r];
      }
  }
}

// The small layer matrices: 16-token x 16-row tiles on v_mfma_f32_16x16x4_f32
// (A = 16 tokens x 4 k, B = 4 k x 16 rows), four waves splitting the blocks
// as above.  A 32 x 32 tile leaves most CUs idle on these shapes and makes
// one wave run a chain of 16 fp32 MFMAs of 64 cycles per block; a 16 x 16 tile
// needs 8 of 32 cycles, and four times as many workgroups share the CUs.
// Within a block, lane quarter kq (= lane / 16) supplies elements 8 kq .. 8 kq
// + 7 over the block's 8 steps (step s: element 8 kq + s), i.e. 32 contiguous
// activation bytes and nibble bytes 4 kq .. 4 kq + 3, in the same order for A
// and B.
template <bool VEC>
__global__ __launch_bounds__(kGemmThreads) void q4_0_gemm16_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t block_bytes,
    const float *__restrict__ x, uint32_t x_bytes, int m, float *__restrict__ y) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int S = 4;                                             // waves splitting the blocks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tok = blockIdx.y * 16 + r16;                           // A row of this lane
  const int row = blockIdx.x * 16 + r16;                           // B column of this lane
  const __amdgpu_buffer_rsrc_t rx = rsrc_q(x, x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc_q(blocks, block_bytes);
  const uint32_t xrow = tok < m ? (uint32_t)tok * (uint32_t)cols * 4u : kOOBq;
  const uint32_t wrow = row < rows ? (uint32_t)row * (uint32_t)nblk * kQBlockBytes : kOOBq;

  struct In {
    float a[8];
    uint32_t nib[2];   // 8 bytes from the aligned address below the lane's 4 nibble bytes
    uint32_t dw;       // the aligned word holding the fp16 scale
  };
  auto load = [&](In &in, int b) {
    const uint32_t xo = xrow + (uint32_t)(kQBlock * b + 8 * kq) * 4u;
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x4q v = __builtin_bit_cast(f32x4q, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16u * i, 0, 0));
        in.a[4 * i + 0] = v.x;
        in.a[4 * i + 1] = v.y;
        in.a[4 * i + 2] = v.z;
        in.a[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        in.a[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, xo + 4u * i, 0, 0));
    }
    const uint32_t bo = wrow + (uint32_t)b * kQBlockBytes;
    in.dw = __builtin_amdgcn_raw_buffer_load_b32(rw, bo & ~3u, 0, 0);
    // two single-word loads: each is range-checked on its own, so a word past
    // the end of the blocks reads 0 (and is then not among the bytes used)
    const uint32_t no = (bo + 2u + 4u * kq) & ~3u;
    in.nib[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, no, 0, 0);
    in.nib[1] = __builtin_amdgcn_raw_buffer_load_b32(rw, no + 4u, 0, 0);
  };
  f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto multiply = [&](In &in, int b) {
    if (b == nblk - 1 && (cols & (kQBlock - 1))) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (kQBlock * b + 8 * kq + s >= cols) in.a[s] = 0.0f;
    }
    const uint32_t bo = wrow + (uint32_t)b * kQBlockBytes;
    const float d = half_bits_to_float((uint16_t)(in.dw >> ((bo & 2u) * 8u)));
    const uint32_t q = __builtin_amdgcn_alignbyte(in.nib[1], in.nib[0], (bo + 2u + 4u * kq) & 3u) ^ 0x88888888u;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int v = __builtin_amdgcn_sbfe((int)q, 4 * s, 4);         // nibble - 8
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(in.a[s], (float)v * d, acc, 0, 0, 0);
    }
  };
  const int last = nblk - 1, kw = wave;
  In in0, in1;
  load(in0, kw < nblk ? kw : last);
  for (int b = kw; b < nblk; b += 2 * S) {
    load(in1, b + S < nblk ? b + S : last);
    __builtin_amdgcn_sched_barrier(0);
    multiply(in0, b);
    __builtin_amdgcn_sched_barrier(0);
    if (b + S < nblk) {                          // uniform
      load(in0, b + 2 * S < nblk ? b + 2 * S : last);
      __builtin_amdgcn_sched_barrier(0);
      multiply(in1, b + S);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // waves 1..3 hand their sums to wave 0, which adds them in wave order
  __shared__ float part[S - 1][4][64];
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < S - 1; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += part[w][r][lane];
  // lane (r16, kq) holds weight row r16 of the tile for tokens 4 kq + r
  if (row < rows) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = blockIdx.y * 16 + 4 * kq + r;
      if (t < m) y[(size_t)t * rows + row] = acc[r];
    }
  }
}

}  // namespace

hipError_t launch_q4_0_gemm(const uint8_t *blocks, int rows, int cols, const float *x, int m,
                            float *y, int num_cus, hipStream_t s) {
  const int nblk = (cols + kQBlock - 1) / kQBlock;
  const size_t block_bytes = (size_t)rows * nblk * kQBlockBytes;
  const size_t x_bytes = (size_t)m * cols * 4;
  if (block_bytes >= ((size_t)1 << 31) || x_bytes >= ((size_t)1 << 31))
    return hipErrorInvalidValue;                 // 32-bit buffer offsets
  // 64 x 64 tiles while they give every CU work, else 32 x 32 tiles with the
  // blocks split over the four waves
  const long big = (long)((rows + kTileN - 1) / kTileN) * ((m + kTileM - 1) / kTileM);
  const bool split = big < num_cus && nblk > 1;
  // 16 x 16 tiles for short rows (at most 16 blocks) while they stay within
  // five workgroups a CU; past that, or for longer rows, the 32 x 32 tiles'
  // fewer activation re-reads win (measured at 512 tokens: 104 x 312 3.4
  // against 5.4 us, 312 x 312 4.9 against 5.5, 520 x 312 6.9 against 7.6;
  // but 1092 x 312 10.9 against 9.4 and 312 x 1092 11.1 against 10.1)
  const long t16n = (long)((rows + 15) / 16) * ((m + 15) / 16);
  const bool t16 = split && nblk <= 16 && t16n <= 5L * num_cus;
  const int tm = split ? 32 : kTileM, tn = split ? 32 : kTileN;
  const dim3 grid((rows + tn - 1) / tn, (m + tm - 1) / tm);
  if (grid.y > 65535) return hipErrorInvalidValue;
  // the blocks' range in whole dwords: a dword load that reaches past the
  // range reads zero as a whole, which would drop the last 2 nibble bytes of
  // the last block when it starts 4-byte aligned (the 1-3 bytes beyond share
  // a dword, hence a page, with the last valid bytes and are never used)
  const uint32_t range = (uint32_t)((block_bytes + 3) & ~(size_t)3);
  auto go = [&](auto kern) {
    kern<<<grid, kGemmThreads, 0, s>>>(blocks, rows, cols, nblk, range, x, (uint32_t)x_bytes, m, y);
  };
  if (t16) {
    const dim3 g16((rows + 15) / 16, (m + 15) / 16);
    if (g16.y > 65535) return hipErrorInvalidValue;
    if ((cols & 3) == 0)
      q4_0_gemm16_kernel<true><<<g16, kGemmThreads, 0, s>>>(blocks, rows, cols, nblk, range, x, (uint32_t)x_bytes, m, y);
    else
      q4_0_gemm16_kernel<false><<<g16, kGemmThreads, 0, s>>>(blocks, rows, cols, nblk, range, x, (uint32_t)x_bytes, m, y);
    return hipGetLastError();
  }
  if ((cols & 3) == 0) {
    if (split) go(q4_0_gemm_kernel<true, 4>);
    else go(q4_0_gemm_kernel<true, 1>);
  } else {
    if (split) go(q4_0_gemm_kernel<false, 4>);
    else go(q4_0_gemm_kernel<false, 1>);
  }
  return hipGetLastError();
}

}  // namespace bqm
