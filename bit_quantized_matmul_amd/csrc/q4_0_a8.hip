// Q4_0 weights against int8 activations (A8): decode GEMV and prefill GEMM.
//
// Minueza-32M -> KMCU v1 page, sections 2 and 3: the 18-byte Q4_0 blocks
// (weight = (nibble - 8) * d, rows padded to whole blocks).  "14MB holds 45M
// parameters" (Needle article), section 1: 8-bit activations; here the
// per-token symmetric codes of act_fwht_quant_a8 with group 1 (no rotation:
// Q4_0 carries none).  Both kernels compute
//   y[t, r] = s[t] * sum_blk fp32(d[r, blk]) * isum(t, r, blk),
//   isum    = sum_{j<32} (nib[r, blk, j] - 8) * q[t, 32 blk + j]   (exact int32)
// so the products are exact integers, each block's sum is scaled by its fp32
// scale once and the blocks are summed in fp32.  Columns >= cols are padding
// with weight 0, so whatever code sits there adds nothing.
//
// GEMV (v_dot4_i32_i8): P = 4..64 lanes share a row, one block each per
// column chunk, as in the fp32 Q4_0 GEMV.  The workgroup stages the chunk's
// codes in LDS once for all its rows, rearranged per 8 codes into the even
// and the odd ones (one v_perm each) with the block's code sum beside them;
// a lane then takes the low and the high nibbles of each nibble word as they
// are (nibble values 0..15) and forms sum nib * q - 8 * sum q, which is the
// block's sum of (nib - 8) * q.
//
// GEMM (v_mfma_i32_32x32x32_i8): one 32-column block per instruction.  Lane
// half h supplies elements 16h .. 16h + 15 of the block to both operands, in
// the same order (the contraction does not depend on how k is ordered, only
// that A and B agree): the codes rearranged to evens then odds of each 8, the
// weights as the low then the high nibbles of each nibble word, each turned
// into the signed byte nibble - 8.  The int32 result of a block is scaled by
// the lane's row scale d and added in fp32; tiles and the split of the
// blocks over waves follow the fp32 Q4_0 GEMM, with 16 x 16 tiles on
// v_mfma_i32_16x16x32_i8 for the short rows of the small layer matrices.
#include "bqm_common.h"
#include "q4_0_block.h"

namespace bqm {
namespace {

constexpr int kA8Threads = 256;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16a __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));

// codes 0..7 of a group (dwords d0 = q0..q3, d1 = q4..q7) -> (q0, q2, q4, q6)
// and (q1, q3, q5, q7)
__device__ __forceinline__ uint32_t evens(uint32_t d1, uint32_t d0) { return __builtin_amdgcn_perm(d1, d0, 0x06040200u); }
__device__ __forceinline__ uint32_t odds(uint32_t d1, uint32_t d0) { return __builtin_amdgcn_perm(d1, d0, 0x07050301u); }

// four nibbles in the low halves of the bytes of t (0..15 each) -> the signed
// bytes nibble - 8: t ^ 8 is nibble - 8 in 4-bit two's complement, and adding
// 0xF0 where its bit 3 is set (8 * 30 = 0xF0, no carry out of a byte)
// sign-extends it to 8 bits
__device__ __forceinline__ uint32_t nib_minus8(uint32_t t) {
  const uint32_t u = t ^ 0x08080808u;
  const uint32_t m = u & 0x08080808u;
  return u + (m << 5) - (m << 1);
}

// The codes of token b, columns c .. c + 7, as two dwords; columns past the
// buffer read as zero (buffer range), columns past the row's end belong to
// the next token but meet zero weights.  ALIGNED: cols % 4 == 0.
template <bool ALIGNED>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t rq, uint32_t off, uint32_t &d0, uint32_t &d1) {
  if constexpr (ALIGNED) {
    d0 = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
    d1 = __builtin_amdgcn_raw_buffer_load_b32(rq, off + 4u, 0, 0);
  } else {
    const uint32_t a = off & ~3u, sh = off & 3u;
    const uint32_t w0 = __builtin_amdgcn_raw_buffer_load_b32(rq, a, 0, 0);
    const uint32_t w1 = __builtin_amdgcn_raw_buffer_load_b32(rq, a + 4u, 0, 0);
    const uint32_t w2 = __builtin_amdgcn_raw_buffer_load_b32(rq, a + 8u, 0, 0);
    d0 = __builtin_amdgcn_alignbyte(w1, w0, sh);
    d1 = __builtin_amdgcn_alignbyte(w2, w1, sh);
  }
}

// ------------------------------------------------------------------- GEMV

template <int BATCH, int P, bool ALIGNED>
__global__ __launch_bounds__(kA8Threads) void q4_0_gemv_a8_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t total,
    const int8_t *__restrict__ q, uint32_t q_bytes, int tok0, const float *__restrict__ scale,
    float *__restrict__ y) {
  // q: the whole [batch, cols] code array (16-byte aligned, so an aligned
  // offset is an aligned address); this launch takes tokens tok0 .. tok0 +
  // BATCH - 1; scale and y start at token tok0
  constexpr int RPW = kA8Threads / P;              // rows per workgroup
  // per token and block of the chunk: 8 dwords (evens, odds of each 8 codes)
  __shared__ __align__(16) uint32_t xs[BATCH][P * 8];
  __shared__ int xsum[BATCH][P];
  const int t = threadIdx.x;
  const int j = t % P;
  const int row = blockIdx.x * RPW + t / P;
  const bool rok = row < rows;
  const __amdgpu_buffer_rsrc_t rw = q4_rsrc(blocks, total);
  const __amdgpu_buffer_rsrc_t rq = q4_rsrc(q, q_bytes);
  float acc[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
  for (int c0 = 0; c0 < nblk; c0 += P) {
    const int blk = c0 + j;
    const bool ok = rok && blk < nblk;
    const BlockLoad L = load_block(rw, ok, ok ? (uint32_t)(((size_t)row * nblk + blk) * kQ4BlockBytes) : 0u, total);
    if (c0 > 0) __syncthreads();                  // the previous chunk's reads are done
    // stage the chunk: thread g < BATCH * P takes token g / P, block g % P
    for (int g = t; g < BATCH * P; g += kA8Threads) {
      const int b = g / P, bi = g - b * P;
      const int col = kQ4Block * (c0 + bi);
      const bool in = c0 + bi < nblk;
      const uint32_t base = (uint32_t)(tok0 + b) * (uint32_t)cols + (uint32_t)col;
      int sum = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t d0, d1;
        load8<ALIGNED>(rq, in ? base + 8u * w : kQ4OOB, d0, d1);
        const uint32_t e = evens(d1, d0), o = odds(d1, d0);
        xs[b][bi * 8 + 2 * w] = e;
        xs[b][bi * 8 + 2 * w + 1] = o;
        sum = __builtin_amdgcn_sdot4((int)e, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)o, 0x01010101, sum, false);
      }
      xsum[b][bi] = sum;
    }
    __syncthreads();
    uint32_t nib[4];
    const float d = block_fields(L, nib);
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const uint4 x0 = *reinterpret_cast<const uint4 *>(&xs[b][j * 8]);
      const uint4 x1 = *reinterpret_cast<const uint4 *>(&xs[b][j * 8 + 4]);
      const uint32_t xe[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      int isum = -8 * xsum[b][j];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        isum = __builtin_amdgcn_sdot4((int)(nib[w] & 0x0F0F0F0Fu), (int)xe[2 * w], isum, false);
        isum = __builtin_amdgcn_sdot4((int)((nib[w] >> 4) & 0x0F0F0F0Fu), (int)xe[2 * w + 1], isum, false);
      }
      acc[b] = fmaf(d, (float)isum, acc[b]);        // d = 0 for a lane without a block
    }
  }
  // butterfly over the P lanes of the row (a fixed order: deterministic)
#pragma unroll
  for (int b = 0; b < BATCH; ++b)
#pragma unroll
    for (int o = P / 2; o >= 1; o >>= 1) acc[b] += __shfl_xor(acc[b], o, P);
  if (rok && j == 0) {
#pragma unroll
    for (int b = 0; b < BATCH; ++b) y[(size_t)b * rows + row] = acc[b] * scale[b];
  }
}

template <int BATCH, bool ALIGNED>
hipError_t gemv_batch(const uint8_t *blocks, int rows, int cols, int nblk, uint32_t total, const int8_t *q,
                      uint32_t q_bytes, int tok0, const float *scale, float *y, hipStream_t s) {
  int P = 4;
  while (P < 64 && P < nblk) P *= 2;               // lanes per row: the power of two covering its blocks
  const int grid = (rows + kA8Threads / P - 1) / (kA8Threads / P);
  switch (P) {
#define BQM_A8_CASE(PP)                                                                              \
  case PP:                                                                                           \
    q4_0_gemv_a8_kernel<BATCH, PP, ALIGNED><<<grid, kA8Threads, 0, s>>>(blocks, rows, cols, nblk, total, \
                                                                        q, q_bytes, tok0, scale, y); \
    break;
    BQM_A8_CASE(4) BQM_A8_CASE(8) BQM_A8_CASE(16) BQM_A8_CASE(32) BQM_A8_CASE(64)
#undef BQM_A8_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ fused GEMV
//
// The same GEMV on fp32 activations, their int8 codes formed in the launch
// with act_fwht_quant_a8's group-1 arithmetic: s = RN(amax / 127) (1 for a
// zero token), q = clamp(rint(RN(x / s)), -127, 127).  Every workgroup forms
// all codes of its tokens once, straight into LDS in the staged layout of the
// kernel above (evens and odds of each 8 codes, each block's code sum), then
// runs its rows with no further staging: workgroups loop over row passes.  The
// first pass's blocks are requested first, so their latency overlaps the
// activations'.
// rint(x * rcp(s)) decides a code unless x * rcp(s) lies within 1e-4 of a
// half-integer (its error is below 127 * 2^-22); then RN(x / s) decides it.
constexpr int kA8FusedMaxLds = 60 * 1024;        // codes of the launch's tokens, per workgroup

template <int BATCH, int P>
__global__ __launch_bounds__(kA8Threads) void q4_0_gemv_a8_fused_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t total,
    const float *__restrict__ x, float *__restrict__ y, int8_t *__restrict__ q_out,
    float *__restrict__ scale_out) {
  // x, y, q_out and scale_out start at the launch's first token
  constexpr int RPW = kA8Threads / P;
  extern __shared__ __align__(16) uint32_t dyn[];
  uint32_t *const xs = dyn;                                         // [BATCH][nblk][8]
  int *const xsum = reinterpret_cast<int *>(dyn + BATCH * nblk * 8);   // [BATCH][nblk]
  __shared__ float red[BATCH][kA8Threads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const __amdgpu_buffer_rsrc_t rx = q4_rsrc(x, (uint32_t)(BATCH * cols) * 4u);
  const __amdgpu_buffer_rsrc_t rw = q4_rsrc(blocks, total);
  const int j = t % P;
  // the first row pass's first blocks are requested before anything else, so
  // their latency overlaps the activations' and the codes'
  BlockLoad L0;
  {
    const int row = blockIdx.x * RPW + t / P;
    const bool ok = row < rows && j < nblk;
    L0 = load_block(rw, ok, ok ? (uint32_t)(((size_t)row * nblk + j) * kQ4BlockBytes) : 0u, total);
  }

  // item i: token i / (4 nblk), block (i / 4) % nblk, codes 8 w .. 8 w + 7 of it
  // (w = i % 4; the four of a block are one lane quad); columns >= cols read 0
  const int nitems = BATCH * nblk * 4;
  auto load_item = [&](int i, float (&v)[8]) {
    const int w = i & 3, bb = i >> 2;
    const int b = bb / nblk, c0 = kQ4Block * (bb - b * nblk) + 8 * w;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rx, c0 + e < cols ? (uint32_t)(b * cols + c0 + e) * 4u : kQ4OOB, 0, 0));
  };

  // 1. the tokens' scales, from one pass over the items (a thread's first item
  // stays in registers for step 2)
  float keep[8];
  float m[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) m[b] = 0.0f;
  for (int i = t; i < nitems; i += kA8Threads) {
    float v[8];
    load_item(i, v);
    const int b = (i >> 2) / nblk;
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
    for (int bt = 0; bt < BATCH; ++bt) m[bt] = bt == b ? fmaxf(m[bt], a) : m[bt];
    if (i == t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) keep[e] = v[e];
    }
  }
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    float mb = m[b];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mb = fmaxf(mb, __shfl_xor(mb, o, 64));
    if (lane == 0) red[b][wave] = mb;
  }
  __syncthreads();
  // every thread forms the scales itself (no second barrier)
  float sc[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    float mm = red[b][0];
#pragma unroll
    for (int w = 1; w < kA8Threads / 64; ++w) mm = fmaxf(mm, red[b][w]);
    sc[b] = mm > 0.0f ? __fdiv_rn(mm, 127.0f) : 1.0f;
  }
  if (scale_out && blockIdx.x == 0 && t < BATCH) {
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (t == b) scale_out[b] = sc[b];
  }

  // 2. the codes, in the staged layout
  for (int i = t; i < nitems; i += kA8Threads) {       // whole quads share a trip count
    const int w = i & 3, bb = i >> 2;
    const int b = bb / nblk, blk = bb - b * nblk;
    float v[8];
    if (i == t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = keep[e];
    } else {
      load_item(i, v);
    }
    float s = sc[0];
#pragma unroll
    for (int bt = 1; bt < BATCH; ++bt) s = b == bt ? sc[bt] : s;
    const float inv = __builtin_amdgcn_rcpf(s);
    const int c0 = kQ4Block * blk + 8 * w;
    int c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = rintf(v[e] * inv);
      if (fabsf(fmaf(v[e], inv, -r)) > 0.4999f) r = rintf(__fdiv_rn(v[e], s));
      c[e] = (int)__builtin_amdgcn_fmed3f(r, -127.0f, 127.0f);
      if (q_out && blockIdx.x == 0 && c0 + e < cols) q_out[(size_t)b * cols + c0 + e] = (int8_t)c[e];
    }
    // evens (codes 0, 2, 4, 6) and odds, one byte each
    const uint32_t e01 = __builtin_amdgcn_perm((uint32_t)c[2], (uint32_t)c[0], 0x0C0C0400u);
    const uint32_t e23 = __builtin_amdgcn_perm((uint32_t)c[6], (uint32_t)c[4], 0x0C0C0400u);
    const uint32_t o01 = __builtin_amdgcn_perm((uint32_t)c[3], (uint32_t)c[1], 0x0C0C0400u);
    const uint32_t o23 = __builtin_amdgcn_perm((uint32_t)c[7], (uint32_t)c[5], 0x0C0C0400u);
    const uint32_t ev = __builtin_amdgcn_perm(e23, e01, 0x05040100u);
    const uint32_t od = __builtin_amdgcn_perm(o23, o01, 0x05040100u);
    *reinterpret_cast<uint2 *>(&xs[(b * nblk + blk) * 8 + 2 * w]) = make_uint2(ev, od);
    int sum = __builtin_amdgcn_sdot4((int)ev, 0x01010101, 0, false);
    sum = __builtin_amdgcn_sdot4((int)od, 0x01010101, sum, false);
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    if (w == 0) xsum[b * nblk + blk] = sum;
  }
  __syncthreads();

  // 3. rows: P lanes a row, RPW rows a pass, the workgroups taking the passes in turn
  bool first = true;
  for (int r0 = blockIdx.x * RPW; r0 < rows; r0 += gridDim.x * RPW) {
    const int row = r0 + t / P;
    const bool rok = row < rows;
    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
    for (int c0 = 0; c0 < nblk; c0 += P) {
      const int blk = c0 + j;
      const bool ok = rok && blk < nblk;
      BlockLoad L;
      if (first) {
        L = L0;
        first = false;
      } else {
        L = load_block(rw, ok, ok ? (uint32_t)(((size_t)row * nblk + blk) * kQ4BlockBytes) : 0u, total);
      }
      uint32_t nib[4];
      const float d = block_fields(L, nib);          // 0 for a lane without a block
      const int bk = blk < nblk ? blk : 0;
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const uint4 x0 = *reinterpret_cast<const uint4 *>(&xs[(b * nblk + bk) * 8]);
        const uint4 x1 = *reinterpret_cast<const uint4 *>(&xs[(b * nblk + bk) * 8 + 4]);
        const uint32_t xe[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        int isum = -8 * xsum[b * nblk + bk];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          isum = __builtin_amdgcn_sdot4((int)(nib[w] & 0x0F0F0F0Fu), (int)xe[2 * w], isum, false);
          isum = __builtin_amdgcn_sdot4((int)((nib[w] >> 4) & 0x0F0F0F0Fu), (int)xe[2 * w + 1], isum, false);
        }
        acc[b] = fmaf(d, (float)isum, acc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
#pragma unroll
      for (int o = P / 2; o >= 1; o >>= 1) acc[b] += __shfl_xor(acc[b], o, P);
    if (rok && j == 0) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) y[(size_t)b * rows + row] = acc[b] * sc[b];
    }
  }
}

template <int BATCH>
hipError_t gemv_fused_batch(const uint8_t *blocks, int rows, int cols, int nblk, uint32_t total, const float *x,
                            float *y, int8_t *q_out, float *scale_out, int num_cus, hipStream_t s) {
  int P = 4;
  while (P < 64 && P < nblk) P *= 2;               // as the staged kernel: the same sums, bit for bit
  const int passes = (rows + kA8Threads / P - 1) / (kA8Threads / P);
  const int grid = passes < 2 * num_cus ? passes : 2 * num_cus;
  const size_t lds = (size_t)BATCH * nblk * 36;
  switch (P) {
#define BQM_A8F_CASE(PP)                                                                                 \
  case PP:                                                                                               \
    q4_0_gemv_a8_fused_kernel<BATCH, PP><<<grid, kA8Threads, lds, s>>>(blocks, rows, cols, nblk, total, x, \
                                                                       y, q_out, scale_out);           \
    break;
    BQM_A8F_CASE(4) BQM_A8F_CASE(8) BQM_A8F_CASE(16) BQM_A8F_CASE(32) BQM_A8F_CASE(64)
#undef BQM_A8F_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------- GEMM

constexpr int kA8TileM = 64, kA8TileN = 64;       // tokens x weight rows per workgroup (KSPLIT 1)

struct A8BlockIn {
  u32x4a a;          // 16 code bytes from the aligned address below the lane's 16,
  uint32_t a4;       // and the next 4
  u32x4a w;          // 16 block bytes from the aligned word below the block, + 8 h
};

// KSPLIT: 1 (2 x 2 wave tiles of 32 x 32) or 4 (one 32 x 32 tile, the blocks
// split over the four waves and summed in LDS in wave order)
template <int KSPLIT>
__global__ __launch_bounds__(kA8Threads) void q4_0_gemm_a8_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t block_bytes,
    const int8_t *__restrict__ q, uint32_t q_bytes, const float *__restrict__ scale, int m,
    float *__restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  constexpr int TM = KSPLIT == 1 ? kA8TileM : 32, TN = KSPLIT == 1 ? kA8TileN : 32;
  const int wm = KSPLIT == 1 ? (wave & 1) : 0, wn = KSPLIT == 1 ? (wave >> 1) : 0;
  const int kw = KSPLIT == 1 ? 0 : wave;                           // first block of this wave
  const int tok = blockIdx.y * TM + 32 * wm + l32;                 // A row of this lane
  const int row = blockIdx.x * TN + 32 * wn + l32;                 // B column of this lane
  const __amdgpu_buffer_rsrc_t rq = q4_rsrc(q, q_bytes);
  const __amdgpu_buffer_rsrc_t rw = q4_rsrc(blocks, block_bytes);
  const uint32_t qrow = tok < m ? (uint32_t)tok * (uint32_t)cols : kQ4OOB;
  const uint32_t wrow = row < rows ? (uint32_t)row * (uint32_t)nblk * kQ4BlockBytes : kQ4OOB;

  // three loads a block: 20 code bytes as 16 + 4, and 16 block bytes, so
  // that the loads per MFMA stay few (each load instruction is an address
  // unit pass for the whole wave)
  auto load = [&](A8BlockIn &in, int b) {
    const uint32_t qo = qrow + (uint32_t)(kQ4Block * b + 16 * h);
    const uint32_t qa = qo & ~3u;
    in.a = __builtin_bit_cast(u32x4a, __builtin_amdgcn_raw_buffer_load_b128(rq, qa, 0, 0));
    in.a4 = __builtin_amdgcn_raw_buffer_load_b32(rq, qa + 16u, 0, 0);
    const uint32_t bo = wrow + (uint32_t)b * kQ4BlockBytes;
    in.w = __builtin_bit_cast(u32x4a, __builtin_amdgcn_raw_buffer_load_b128(rw, (bo & ~3u) + 8u * h, 0, 0));
  };

  f32x16a acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  auto multiply = [&](const A8BlockIn &in, int b) {
    // codes 16h .. 16h + 15 of the block, realigned, as evens / odds of each 8
    const uint32_t qo = qrow + (uint32_t)(kQ4Block * b + 16 * h);
    const uint32_t sq = qo & 3u;
    const uint32_t aw[5] = {in.a.x, in.a.y, in.a.z, in.a.w, in.a4};
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_alignbyte(aw[i + 1], aw[i], sq);
    const i32x4 A = {(int)evens(c[1], c[0]), (int)odds(c[1], c[0]), (int)evens(c[3], c[2]), (int)odds(c[3], c[2])};
    // nibble bytes 8h .. 8h + 7 (elements 16h ..), at byte (bo & 3) + 2 of the
    // lane's window (2 or 4: blocks are 2-byte aligned), realigned; low
    // nibbles are the even elements, high nibbles the odd ones.  The scale
    // sits in the first word of the lower half's window; lane l32 + 32 (the
    // same weight row) takes it from lane l32.
    const uint32_t bo = wrow + (uint32_t)b * kQ4BlockBytes;
    const uint32_t dlo = (uint32_t)__shfl_xor((int)in.w.x, 32, 64);
    const float d = half_bits_to_float((uint16_t)((h ? dlo : in.w.x) >> ((bo & 2u) * 8u)));
    const bool at4 = (bo & 2u) != 0;                 // nibbles start at byte 4: word 1
    const uint32_t w0 = at4 ? in.w.y : in.w.x, w1 = at4 ? in.w.z : in.w.y, w2 = at4 ? in.w.w : in.w.z;
    const uint32_t n0 = __builtin_amdgcn_alignbyte(w1, w0, at4 ? 0u : 2u);
    const uint32_t n1 = __builtin_amdgcn_alignbyte(w2, w1, at4 ? 0u : 2u);
    const i32x4 Bv = {(int)nib_minus8(n0 & 0x0F0F0F0Fu), (int)nib_minus8((n0 >> 4) & 0x0F0F0F0Fu),
                      (int)nib_minus8(n1 & 0x0F0F0F0Fu), (int)nib_minus8((n1 >> 4) & 0x0F0F0F0Fu)};
    i32x16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0;
    const i32x16 isum = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bv, zero, 0, 0, 0);
    // lane (l32, h) holds column l32 (its own weight row, scale d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = fmaf(d, (float)isum[r], acc[r]);
  };
  // two buffers in turn: block b + S's loads go out before block b is
  // multiplied; loads past the wave's last block read the last block again
  // and are not used
  constexpr int S = KSPLIT;
  const int last = nblk - 1;
  A8BlockIn in0, in1;
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
  // lane (l32, h) holds weight row l32 of the wave tile's columns and tokens
  // 8 i + 4 h + r (i, r < 4) of its rows
  if (row < rows) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = blockIdx.y * TM + 32 * wm + 8 * i + 4 * h + r;
        if (tt < m) y[(size_t)tt * rows + row] = acc[4 * i + r] * scale[tt];
      }
  }
}

// The small layer matrices: 16-token x 16-row tiles on v_mfma_i32_16x16x32_i8,
// one block per instruction, the blocks split over the four waves as above.
// Lane quarter kq (= lane / 16) supplies elements 8 kq .. 8 kq + 7 of a block
// to both operands in the same order: the 8 codes as evens then odds, the 4
// nibble bytes 4 kq .. 4 kq + 3 as their low then their high nibbles, each
// turned into nibble - 8.  The int32 result of a block is scaled by the row's d
// and added in fp32, as in the 32 x 32 kernel.  ALIGNED: cols % 4 == 0.
template <bool ALIGNED>
__global__ __launch_bounds__(kA8Threads) void q4_0_gemm_a8_16_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t block_bytes,
    const int8_t *__restrict__ q, uint32_t q_bytes, const float *__restrict__ scale, int m,
    float *__restrict__ y) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int S = 4;                                             // waves splitting the blocks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tok = blockIdx.y * 16 + r16;                           // A row of this lane
  const int row = blockIdx.x * 16 + r16;                           // B column of this lane
  const __amdgpu_buffer_rsrc_t rq = q4_rsrc(q, q_bytes);
  const __amdgpu_buffer_rsrc_t rw = q4_rsrc(blocks, block_bytes);
  const uint32_t qrow = tok < m ? (uint32_t)tok * (uint32_t)cols : kQ4OOB;
  const uint32_t wrow = row < rows ? (uint32_t)row * (uint32_t)nblk * kQ4BlockBytes : kQ4OOB;

  struct In {
    uint32_t c0, c1;   // codes 8 kq .. 8 kq + 7 of the block
    uint32_t n0, n1;   // the two words from the aligned address below the lane's nibble bytes
    uint32_t dw;       // the aligned word holding the fp16 scale
  };
  auto load = [&](In &in, int b) {
    load8<ALIGNED>(rq, qrow + (uint32_t)(kQ4Block * b + 8 * kq), in.c0, in.c1);
    const uint32_t bo = wrow + (uint32_t)b * kQ4BlockBytes;
    in.dw = __builtin_amdgcn_raw_buffer_load_b32(rw, bo & ~3u, 0, 0);
    // single-word loads: a word past the end of the blocks reads 0 on its own
    // (and is then not among the bytes used)
    const uint32_t no = (bo + 2u + 4u * kq) & ~3u;
    in.n0 = __builtin_amdgcn_raw_buffer_load_b32(rw, no, 0, 0);
    in.n1 = __builtin_amdgcn_raw_buffer_load_b32(rw, no + 4u, 0, 0);
  };
  f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto multiply = [&](const In &in, int b) {
    const uint32_t bo = wrow + (uint32_t)b * kQ4BlockBytes;
    const float d = half_bits_to_float((uint16_t)(in.dw >> ((bo & 2u) * 8u)));
    const uint32_t n = __builtin_amdgcn_alignbyte(in.n1, in.n0, (bo + 2u + 4u * kq) & 3u);
    const uint64_t a = (uint64_t)evens(in.c1, in.c0) | ((uint64_t)odds(in.c1, in.c0) << 32);
    const uint64_t w = (uint64_t)nib_minus8(n & 0x0F0F0F0Fu) | ((uint64_t)nib_minus8((n >> 4) & 0x0F0F0F0Fu) << 32);
    const i32x4 zero = {0, 0, 0, 0};
    const i32x4 isum = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)w, zero, 0, 0, 0);
    // lane (r16, kq) holds column r16 (its own weight row, scale d)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(d, (float)isum[r], acc[r]);
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
      if (t < m) y[(size_t)t * rows + row] = acc[r] * scale[t];
    }
  }
}

}  // namespace

hipError_t launch_q4_0_gemv_a8(const uint8_t *blocks, int rows, int cols, const int8_t *q,
                               const float *scale, int batch, float *y, hipStream_t s) {
  const int nblk = (cols + kQ4Block - 1) / kQ4Block;
  const size_t total = (size_t)rows * nblk * kQ4BlockBytes;
  // the codes' range in whole dwords (a dword load reaching past the range
  // reads zero as a whole; the 1-3 bytes beyond share a dword, hence a page,
  // with the last valid code and meet zero weights)
  const uint32_t qbytes = (uint32_t)(((size_t)batch * cols + 3) & ~(size_t)3);
  for (int b0 = 0; b0 < batch;) {
    const int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    float *yb = y + (size_t)b0 * rows;
    const float *sb = scale + b0;
    const bool al = (cols & 3) == 0;
    const uint32_t tb = (uint32_t)total;
    hipError_t e;
    if (nb == 4) e = al ? gemv_batch<4, true>(blocks, rows, cols, nblk, tb, q, qbytes, b0, sb, yb, s)
                        : gemv_batch<4, false>(blocks, rows, cols, nblk, tb, q, qbytes, b0, sb, yb, s);
    else if (nb == 2) e = al ? gemv_batch<2, true>(blocks, rows, cols, nblk, tb, q, qbytes, b0, sb, yb, s)
                             : gemv_batch<2, false>(blocks, rows, cols, nblk, tb, q, qbytes, b0, sb, yb, s);
    else e = al ? gemv_batch<1, true>(blocks, rows, cols, nblk, tb, q, qbytes, b0, sb, yb, s)
                : gemv_batch<1, false>(blocks, rows, cols, nblk, tb, q, qbytes, b0, sb, yb, s);
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

// tokens a launch: 4, 2 or 1, as many as the remaining batch and the LDS allow
static int fused_slice(int remaining, int nblk) {
  for (int nb = 4; nb > 1; nb >>= 1)
    if (remaining >= nb && (size_t)nb * nblk * 36 <= (size_t)kA8FusedMaxLds) return nb;
  return 1;
}

bool q4_0_gemv_a8_fused_supported(int cols, int batch) {
  const size_t nblk = ((size_t)cols + kQ4Block - 1) / kQ4Block;
  return (size_t)batch * cols < ((size_t)1 << 29) && nblk * 36 <= (size_t)kA8FusedMaxLds;
}

hipError_t launch_q4_0_gemv_a8_fused(const uint8_t *blocks, int rows, int cols, const float *x, int batch,
                                     float *y, int8_t *q_out, float *scale_out, int num_cus, hipStream_t s) {
  const int nblk = (cols + kQ4Block - 1) / kQ4Block;
  const uint32_t total = (uint32_t)((size_t)rows * nblk * kQ4BlockBytes);
  for (int b0 = 0; b0 < batch;) {
    const int nb = fused_slice(batch - b0, nblk);
    const float *xb = x + (size_t)b0 * cols;
    float *yb = y + (size_t)b0 * rows;
    int8_t *qb = q_out ? q_out + (size_t)b0 * cols : nullptr;
    float *sb = scale_out ? scale_out + b0 : nullptr;
    hipError_t e;
    if (nb == 4) e = gemv_fused_batch<4>(blocks, rows, cols, nblk, total, xb, yb, qb, sb, num_cus, s);
    else if (nb == 2) e = gemv_fused_batch<2>(blocks, rows, cols, nblk, total, xb, yb, qb, sb, num_cus, s);
    else e = gemv_fused_batch<1>(blocks, rows, cols, nblk, total, xb, yb, qb, sb, num_cus, s);
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

hipError_t launch_q4_0_gemm_a8(const uint8_t *blocks, int rows, int cols, const int8_t *q, const float *scale,
                               int m, float *y, int num_cus, hipStream_t s) {
  const int nblk = (cols + kQ4Block - 1) / kQ4Block;
  // ranges in whole dwords (see launch_q4_0_gemv_a8; for the blocks, the
  // last block's nibble load would otherwise lose its last 2 bytes when the
  // block starts 4-byte aligned)
  const size_t block_bytes = ((size_t)rows * nblk * kQ4BlockBytes + 3) & ~(size_t)3;
  const size_t q_bytes = ((size_t)m * cols + 3) & ~(size_t)3;
  // 64 x 64 tiles while they give every CU work, else 32 x 32 tiles with the
  // blocks split over the four waves
  const long big = (long)((rows + kA8TileN - 1) / kA8TileN) * ((m + kA8TileM - 1) / kA8TileM);
  const bool split = big < num_cus && nblk > 1;
  const int tm = split ? 32 : kA8TileM, tn = split ? 32 : kA8TileN;
  const dim3 grid((rows + tn - 1) / tn, (m + tm - 1) / tm);
  // 16 x 16 tiles for short rows (at most 16 blocks) while they stay within
  // five workgroups a CU, as in the fp32 Q4_0 GEMM (measured at 512 tokens:
  // 104 x 312 3.3 against 5.1 us, 312 x 312 4.3 against 5.2; 1092 x 312 8.1
  // against 6.5 and 312 x 1092 8.0 against 7.3 with them, so those keep 32 x 32)
  const long t16n = (long)((rows + 15) / 16) * ((m + 15) / 16);
  const bool t16 = split && nblk <= 16 && t16n <= 5L * num_cus;
  if (t16) {
    const dim3 g16((rows + 15) / 16, (m + 15) / 16);
    if ((cols & 3) == 0)
      q4_0_gemm_a8_16_kernel<true><<<g16, kA8Threads, 0, s>>>(blocks, rows, cols, nblk, (uint32_t)block_bytes, q,
                                                               (uint32_t)q_bytes, scale, m, y);
    else
      q4_0_gemm_a8_16_kernel<false><<<g16, kA8Threads, 0, s>>>(blocks, rows, cols, nblk, (uint32_t)block_bytes, q,
                                                                (uint32_t)q_bytes, scale, m, y);
    return hipGetLastError();
  }
  if (split)
    q4_0_gemm_a8_kernel<4><<<grid, kA8Threads, 0, s>>>(blocks, rows, cols, nblk, (uint32_t)block_bytes, q,
                                                       (uint32_t)q_bytes, scale, m, y);
  else
    q4_0_gemm_a8_kernel<1><<<grid, kA8Threads, 0, s>>>(blocks, rows, cols, nblk, (uint32_t)block_bytes, q,
                                                       (uint32_t)q_bytes, scale, m, y);
  return hipGetLastError();
}

}  // namespace bqm
