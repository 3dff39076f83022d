// Q4_0 GEMV and Q4_0 encoder.
//
// Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html):
//  section 2: 32 weights per 18-byte block, fp16 scale d = max|w|/8 in bytes
//  [0,2), then 16 bytes of 4-bit codes q+8 with the low nibble holding the
//  even element; a weight decodes as (nibble - 8) * d.
//  section 3: each row is zero-padded to a multiple of 32, so a row owns
//  ceil(cols/32) whole blocks and the GEMV inner loop has a fixed length 32.
//
// GEMV: y[b, r] = sum_blk fp32(d[r, blk]) * sum_{j<32} (nib[r, blk, j] - 8) * x[b, 32 blk + j],
// columns >= cols are padding (weight 0) and x is taken as 0 there.
// Decode matrices are small (a few hundred KB), so the kernel is built for
// latency: P = 4..64 lanes of one wave share a row, one 18-byte block each per
// P-block column chunk; every lane issues its weight loads before anything
// else, the workgroup stages the chunk of x in LDS meanwhile, and the row sum
// closes with a butterfly across the P lanes (no LDS, no second barrier).
// An 18-byte block is fetched as the 16 bytes from the 4-byte-aligned address
// below it plus the next 4 (2 for a final block that ends there), then
// realigned with v_alignbyte.  Rows of 9 to 16 blocks (every Minueza matrix
// but the down projections) take a second kernel with no LDS and no barrier:
// 16 lanes a row, each lane's activations in registers, row tiles walked by a
// persistent grid (q4_0_gemv_rows_kernel below).
#include "bqm_common.h"
#include "q4_0_block.h"

namespace bqm {
namespace {

constexpr int kThreads = 256;
constexpr int kBlock = kQ4Block;
constexpr int kBlockBytes = kQ4BlockBytes;

// Byte K of v as a float; matches v_cvt_f32_ubyteK.
template <int K>
__device__ __forceinline__ float ubyte_f(uint32_t v) { return (float)((v >> (8 * K)) & 0xFFu); }

// Rotation by R lanes inside each 16-lane DPP row (row_ror:R).
template <int R>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + R,
                                                                 0xF, 0xF, false));
}

// acc[b] += d * sum_{j<32} (nib_j - 8) * x[b][e0 + j] for the loaded block,
// x from the LDS copy xs (row stride XS floats).
template <int BATCH, int XS>
__device__ __forceinline__ void block_dot(const BlockLoad &L, const float (*xs)[XS], int e0,
                                          float (&acc)[BATCH]) {
  uint32_t nib[4];                                 // byte k of nib[w]: elements 8w+2k (low), 8w+2k+1 (high)
  const float d = block_fields(L, nib);
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 xa = *reinterpret_cast<const float4 *>(&xs[b][e0 + 8 * w]);
      const float4 xc = *reinterpret_cast<const float4 *>(&xs[b][e0 + 8 * w + 4]);
      const uint32_t lo = nib[w] & 0x0F0F0F0Fu;
      const uint32_t hi = (nib[w] >> 4) & 0x0F0F0F0Fu;
      s0 = fmaf(ubyte_f<0>(lo) - 8.0f, xa.x, s0);
      s1 = fmaf(ubyte_f<0>(hi) - 8.0f, xa.y, s1);
      s0 = fmaf(ubyte_f<1>(lo) - 8.0f, xa.z, s0);
      s1 = fmaf(ubyte_f<1>(hi) - 8.0f, xa.w, s1);
      s0 = fmaf(ubyte_f<2>(lo) - 8.0f, xc.x, s0);
      s1 = fmaf(ubyte_f<2>(hi) - 8.0f, xc.y, s1);
      s0 = fmaf(ubyte_f<3>(lo) - 8.0f, xc.z, s0);
      s1 = fmaf(ubyte_f<3>(hi) - 8.0f, xc.w, s1);
    }
    acc[b] = fmaf(d, s0 + s1, acc[b]);
  }
}

// x [BATCH, cols] columns [col0, col0 + n) to xs, zeros past cols.
template <int BATCH, int XS>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int cols, int col0, bool vec,
                                        float (*xs)[XS]) {
  const int ncol = min(XS, cols - col0);
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    const float *xb = x + (size_t)b * cols + col0;
    for (int e = threadIdx.x * 4; e < XS; e += kThreads * 4) {
      float4 q = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (vec && e + 3 < ncol) {
        q = *reinterpret_cast<const float4 *>(xb + e);
      } else {
        if (e < ncol) q.x = xb[e];
        if (e + 1 < ncol) q.y = xb[e + 1];
        if (e + 2 < ncol) q.z = xb[e + 2];
        if (e + 3 < ncol) q.w = xb[e + 3];
      }
      *reinterpret_cast<float4 *>(&xs[b][e]) = q;
    }
  }
}

template <int BATCH, int P>
__global__ __launch_bounds__(kThreads) void q4_0_gemv_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t total,
    const float *__restrict__ x, float *__restrict__ y) {
  constexpr int RPW = kThreads / P;        // rows per workgroup
  constexpr int kChunk = P;                // blocks per column chunk: one per lane
  __shared__ __align__(16) float xs[BATCH][kChunk * kBlock];
  const int t = threadIdx.x;
  const int j = t % P;
  const int row = blockIdx.x * RPW + t / P;
  const bool rok = row < rows;
  const __amdgpu_buffer_rsrc_t rw = q4_rsrc(blocks, total);
  const bool vec = ((cols & 3) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  float acc[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
  for (int c0 = 0; c0 < nblk; c0 += kChunk) {
    // the lane's block c0 + j: its loads first (out of range reads 0)
    const int blk = c0 + j;
    const bool ok = rok && blk < nblk;
    const BlockLoad L = load_block(rw, ok, ok ? (uint32_t)(((size_t)row * nblk + blk) * kBlockBytes) : 0u, total);
    // x columns [32 c0, 32 (c0 + P)) to LDS meanwhile, zero past cols
    if (c0 > 0) __syncthreads();                           // the previous chunk's reads are done
    stage_x<BATCH>(x, cols, c0 * kBlock, vec, xs);
    __syncthreads();
    block_dot<BATCH>(L, xs, j * kBlock, acc);
  }
  // butterfly over the P lanes of the row (a fixed order: deterministic)
#pragma unroll
  for (int b = 0; b < BATCH; ++b)
#pragma unroll
    for (int o = P / 2; o >= 1; o >>= 1) acc[b] += __shfl_xor(acc[b], o, P);
  if (rok && j == 0) {
#pragma unroll
    for (int b = 0; b < BATCH; ++b) y[(size_t)b * rows + row] = acc[b];
  }
}

// Rows of 9 to 16 blocks: 16 lanes (one DPP row) per matrix row, one block
// each, and the workgroup walks NT row tiles (tiles blockIdx.x + i *
// gridDim.x).  A lane's 32 activations (those of its block column, zero past
// cols) come straight from global memory into registers, ahead of the NT
// tiles' block loads, so there is no LDS staging and no barrier: each tile is
// summed as soon as its loads land.  The row sum closes with the rotations
// by 1, 2, 4, 8 inside the 16-lane row (every lane ends with the total, in
// the same fixed order).  VEC: cols % 4 == 0 and x 16-byte aligned.
typedef uint32_t u32x4q __attribute__((ext_vector_type(4)));
template <int BATCH, int NT, bool VEC>
__global__ __launch_bounds__(kThreads) void q4_0_gemv_rows_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, uint32_t total,
    const float *__restrict__ x, float *__restrict__ y) {
  constexpr int P = 16;
  constexpr int RPW = kThreads / P;        // rows per tile
  const int t = threadIdx.x;
  const int j = t % P;
  const __amdgpu_buffer_rsrc_t rw = q4_rsrc(blocks, total);
  const __amdgpu_buffer_rsrc_t rx = q4_rsrc(x, (uint32_t)((size_t)BATCH * cols * 4));
  // activations of block column j: 8 loads of 4 floats per token (columns
  // past cols read 0: each token's range is checked through its own offset)
  float xr[BATCH][kBlock];
#pragma unroll
  for (int b = 0; b < BATCH; ++b)
#pragma unroll
    for (int u = 0; u < kBlock / 4; ++u) {
      const int c = j * kBlock + 4 * u;
      if constexpr (VEC) {
        const u32x4q v = __builtin_bit_cast(u32x4q, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rx, c < cols ? (uint32_t)((b * cols + c) * 4) : kQ4OOB, 0, 0));
        xr[b][4 * u + 0] = __uint_as_float(v.x);
        xr[b][4 * u + 1] = __uint_as_float(v.y);
        xr[b][4 * u + 2] = __uint_as_float(v.z);
        xr[b][4 * u + 3] = __uint_as_float(v.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xr[b][4 * u + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rx, c + e < cols ? (uint32_t)((b * cols + c + e) * 4) : kQ4OOB, 0, 0));
      }
    }
  BlockLoad L[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int row = (blockIdx.x + i * gridDim.x) * RPW + t / P;
    const bool ok = row < rows && j < nblk;
    L[i] = load_block(rw, ok, ok ? (uint32_t)(((size_t)row * nblk + j) * kBlockBytes) : 0u, total);
  }
  // sum_j (nib_j - 8) x_j = sum_j nib_j x_j - 8 sum_j x_j: the lane's
  // activations are the same for every tile, so their sum is taken once
  // (nib_j x_j is exact; the two sums round like any fp32 reduction)
  float xs8[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int e = 0; e < kBlock; e += 2) {
      a0 += xr[b][e];
      a1 += xr[b][e + 1];
    }
    xs8[b] = 8.0f * (a0 + a1);
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int row = (blockIdx.x + i * gridDim.x) * RPW + t / P;
    uint32_t nib[4];
    const float d = block_fields(L[i], nib);
    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = nib[w] & 0x0F0F0F0Fu;
        const uint32_t hi = (nib[w] >> 4) & 0x0F0F0F0Fu;
        s0 = fmaf(ubyte_f<0>(lo), xr[b][8 * w + 0], s0);
        s1 = fmaf(ubyte_f<0>(hi), xr[b][8 * w + 1], s1);
        s0 = fmaf(ubyte_f<1>(lo), xr[b][8 * w + 2], s0);
        s1 = fmaf(ubyte_f<1>(hi), xr[b][8 * w + 3], s1);
        s0 = fmaf(ubyte_f<2>(lo), xr[b][8 * w + 4], s0);
        s1 = fmaf(ubyte_f<2>(hi), xr[b][8 * w + 5], s1);
        s0 = fmaf(ubyte_f<3>(lo), xr[b][8 * w + 6], s0);
        s1 = fmaf(ubyte_f<3>(hi), xr[b][8 * w + 7], s1);
      }
      float v = d * ((s0 + s1) - xs8[b]);
      v += row_ror<1>(v);
      v += row_ror<2>(v);
      v += row_ror<4>(v);
      v += row_ror<8>(v);
      acc[b] = v;
    }
    if (row < rows && j == 0) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) y[(size_t)b * rows + row] = acc[b];
    }
  }
}

// One thread per block.  fp32 throughout, matching the page's numpy:
// amax = max|w|; d = amax / 8 (1 if amax == 0); q = clip(rint(w / d), -8, 7).
__global__ __launch_bounds__(kThreads) void q4_0_pack_kernel(const float *__restrict__ w, int rows,
                                                            int cols, int nblk,
                                                            uint8_t *__restrict__ out) {
  const long total = (long)rows * nblk;
  for (long g = (long)blockIdx.x * kThreads + threadIdx.x; g < total;
       g += (long)gridDim.x * kThreads) {
    const int row = (int)(g / nblk);
    const int blk = (int)(g - (long)row * nblk);
    const int c0 = blk * kBlock;
    float v[kBlock];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < kBlock; ++e) {
      v[e] = (c0 + e < cols) ? w[(size_t)row * cols + c0 + e] : 0.0f;
      amax = fmaxf(amax, fabsf(v[e]));
    }
    const float d = (amax > 0.0f) ? __fdiv_rn(amax, 8.0f) : 1.0f;
    uint16_t *dst = reinterpret_cast<uint16_t *>(out + (size_t)g * kBlockBytes);
    dst[0] = __builtin_bit_cast(uint16_t, (_Float16)d);   // v_cvt_f16_f32: round to nearest even
#pragma unroll
    for (int k = 0; k < kBlock / 4; ++k) {      // ushort k: elements 4k .. 4k+3
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float r = rintf(__fdiv_rn(v[4 * k + e], d));
        r = fminf(fmaxf(r, -8.0f), 7.0f);
        packed |= (uint32_t)((int)r + 8) << (4 * e);
      }
      dst[1 + k] = (uint16_t)packed;
    }
  }
}

constexpr int kRowsWgPerCu = 2;            // row-tile kernel: workgroups per CU
constexpr int kRowsMaxNT = 8;              // ... and at most this many tiles a workgroup

template <int BATCH, bool VEC>
hipError_t launch_rows(const uint8_t *blocks, int rows, int cols, int nblk, uint32_t total,
                       const float *x, float *y, int num_cus, hipStream_t s) {
  const int tiles = (rows + kThreads / 16 - 1) / (kThreads / 16);
  int grid = num_cus * kRowsWgPerCu;
  if (grid * kRowsMaxNT < tiles) grid = (tiles + kRowsMaxNT - 1) / kRowsMaxNT;
  if (grid > tiles) grid = tiles;
  const int nt = (tiles + grid - 1) / grid;
  if (nt <= 1) q4_0_gemv_rows_kernel<BATCH, 1, VEC><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y);
  else if (nt <= 2) q4_0_gemv_rows_kernel<BATCH, 2, VEC><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y);
  else if (nt <= 4) q4_0_gemv_rows_kernel<BATCH, 4, VEC><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y);
  else q4_0_gemv_rows_kernel<BATCH, 8, VEC><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y);
  return hipGetLastError();
}

template <int BATCH>
hipError_t launch_batch(const uint8_t *blocks, int rows, int cols, int nblk, uint32_t total,
                        const float *x, float *y, int num_cus, hipStream_t s) {
  // lanes per row: the power of two covering the row's blocks (4 .. 64)
  int P = 4;
  while (P < 64 && P < nblk) P *= 2;
  // rows of 9 to 16 blocks: row tiles with the activations in registers (a
  // persistent grid for tall matrices, one tile a workgroup for short ones)
  if (P == 16) {
    const bool vec = ((cols & 3) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    return vec ? launch_rows<BATCH, true>(blocks, rows, cols, nblk, total, x, y, num_cus, s)
               : launch_rows<BATCH, false>(blocks, rows, cols, nblk, total, x, y, num_cus, s);
  }
  const int grid = (rows + kThreads / P - 1) / (kThreads / P);
  switch (P) {
    case 4: q4_0_gemv_kernel<BATCH, 4><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y); break;
    case 8: q4_0_gemv_kernel<BATCH, 8><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y); break;
    case 16: q4_0_gemv_kernel<BATCH, 16><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y); break;
    case 32: q4_0_gemv_kernel<BATCH, 32><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y); break;
    default: q4_0_gemv_kernel<BATCH, 64><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, x, y); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_0_gemv(const uint8_t *blocks, int rows, int cols, const float *x, int batch,
                            float *y, int num_cus, hipStream_t s) {
  const int nblk = (cols + kBlock - 1) / kBlock;
  const size_t total = (size_t)rows * nblk * kBlockBytes;
  if (total >= ((size_t)1 << 31)) return hipErrorInvalidValue;   // 32-bit buffer offsets
  for (int b0 = 0; b0 < batch;) {
    const int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    const float *xb = x + (size_t)b0 * cols;
    float *yb = y + (size_t)b0 * rows;
    hipError_t e;
    if (nb == 4) e = launch_batch<4>(blocks, rows, cols, nblk, (uint32_t)total, xb, yb, num_cus, s);
    else if (nb == 2) e = launch_batch<2>(blocks, rows, cols, nblk, (uint32_t)total, xb, yb, num_cus, s);
    else e = launch_batch<1>(blocks, rows, cols, nblk, (uint32_t)total, xb, yb, num_cus, s);
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

hipError_t launch_q4_0_pack(const float *w, int rows, int cols, uint8_t *blocks, hipStream_t s) {
  const int nblk = (cols + kBlock - 1) / kBlock;
  const long total = (long)rows * nblk;
  long grid = (total + kThreads - 1) / kThreads;
  if (grid > 65535) grid = 65535;
  q4_0_pack_kernel<<<(int)grid, kThreads, 0, s>>>(w, rows, cols, nblk, blocks);
  return hipGetLastError();
}

}  // namespace bqm
