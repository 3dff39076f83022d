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
// columns >= cols are padding (weight 0) and x is never read there.
// A workgroup takes whole rows: `P` threads share a row (one or more blocks
// each), partial sums meet in LDS and one thread per row adds them in a fixed
// order (deterministic).  An 18-byte block is fetched with one 16-byte load
// from the 4-byte-aligned address below it plus one 4-byte load, then
// realigned with v_alignbyte.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads = 256;
constexpr int kBlock = 32;
constexpr int kBlockBytes = 18;

// Byte K of v as a float; matches v_cvt_f32_ubyteK.
template <int K>
__device__ __forceinline__ float ubyte_f(uint32_t v) { return (float)((v >> (8 * K)) & 0xFFu); }

struct Q4Block {
  float d;
  uint32_t nib[4];   // 16 code bytes: byte k of nib[w] holds elements 8w+2k (low), 8w+2k+1 (high)
};

__device__ __forceinline__ Q4Block load_block(const uint8_t *base, size_t off, size_t total) {
  const size_t a4 = off & ~(size_t)3;
  const uint32_t sh = (uint32_t)(off & 3);        // 0 or 2: blocks are 2-byte aligned
  const uint4 v = *reinterpret_cast<const uint4 *>(base + a4);
  uint32_t v4;
  if (a4 + 20 <= total)
    v4 = *reinterpret_cast<const uint32_t *>(base + a4 + 16);
  else
    v4 = (uint32_t)*reinterpret_cast<const uint16_t *>(base + a4 + 16);
  uint32_t w0, w1, w2, w3, w4;
  if (sh == 0) {
    w0 = v.x; w1 = v.y; w2 = v.z; w3 = v.w; w4 = v4;
  } else {
    w0 = __builtin_amdgcn_alignbyte(v.y, v.x, 2);
    w1 = __builtin_amdgcn_alignbyte(v.z, v.y, 2);
    w2 = __builtin_amdgcn_alignbyte(v.w, v.z, 2);
    w3 = __builtin_amdgcn_alignbyte(v4, v.w, 2);
    w4 = v4 >> 16;
  }
  Q4Block b;
  b.d = half_bits_to_float((uint16_t)(w0 & 0xFFFFu));
  b.nib[0] = __builtin_amdgcn_alignbyte(w1, w0, 2);
  b.nib[1] = __builtin_amdgcn_alignbyte(w2, w1, 2);
  b.nib[2] = __builtin_amdgcn_alignbyte(w3, w2, 2);
  b.nib[3] = __builtin_amdgcn_alignbyte(w4, w3, 2);
  return b;
}

template <int BATCH>
__global__ __launch_bounds__(kThreads) void q4_0_gemv_kernel(
    const uint8_t *__restrict__ blocks, int rows, int cols, int nblk, size_t total,
    const float *__restrict__ x, float *__restrict__ y, int P, int R, int bpt) {
  __shared__ float part[BATCH][kThreads];
  const int t = threadIdx.x;
  const int rl = t / P;
  const int j = t - rl * P;
  const bool vec_x = (cols & 3) == 0;
  for (int base = blockIdx.x * R; base < rows; base += gridDim.x * R) {
    const int row = base + rl;
    const bool ok = rl < R && row < rows;
    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
    if (ok) {
      for (int i = 0; i < bpt; ++i) {
        const int blk = j + P * i;
        if (blk >= nblk) break;
        const Q4Block qb = load_block(blocks, ((size_t)row * nblk + blk) * kBlockBytes, total);
        const int c0 = blk * kBlock;
        const int nvalid = min(kBlock, cols - c0);
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          const float *xb = x + (size_t)b * cols + c0;
          float s = 0.0f;
          if (nvalid == kBlock && vec_x) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float4 xa = *reinterpret_cast<const float4 *>(xb + 8 * w);
              const float4 xc = *reinterpret_cast<const float4 *>(xb + 8 * w + 4);
              const uint32_t lo = qb.nib[w] & 0x0F0F0F0Fu;
              const uint32_t hi = (qb.nib[w] >> 4) & 0x0F0F0F0Fu;
              s = fmaf(ubyte_f<0>(lo) - 8.0f, xa.x, s);
              s = fmaf(ubyte_f<0>(hi) - 8.0f, xa.y, s);
              s = fmaf(ubyte_f<1>(lo) - 8.0f, xa.z, s);
              s = fmaf(ubyte_f<1>(hi) - 8.0f, xa.w, s);
              s = fmaf(ubyte_f<2>(lo) - 8.0f, xc.x, s);
              s = fmaf(ubyte_f<2>(hi) - 8.0f, xc.y, s);
              s = fmaf(ubyte_f<3>(lo) - 8.0f, xc.z, s);
              s = fmaf(ubyte_f<3>(hi) - 8.0f, xc.w, s);
            }
          } else {
            for (int e = 0; e < nvalid; ++e) {
              const uint32_t byte = (qb.nib[e >> 3] >> (8 * ((e >> 1) & 3))) & 0xFFu;
              const uint32_t nb = (e & 1) ? (byte >> 4) : (byte & 15u);
              s = fmaf((float)nb - 8.0f, xb[e], s);
            }
          }
          acc[b] = fmaf(qb.d, s, acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) part[b][t] = acc[b];
    __syncthreads();
    if (ok && j == 0) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        float s = 0.0f;
        for (int k = 0; k < P; ++k) s += part[b][rl * P + k];
        y[(size_t)b * rows + row] = s;
      }
    }
    __syncthreads();
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

}  // namespace

hipError_t launch_q4_0_gemv(const uint8_t *blocks, int rows, int cols, const float *x, int batch,
                            float *y, int num_cus, hipStream_t s) {
  const int nblk = (cols + kBlock - 1) / kBlock;
  const int P = nblk < kThreads ? nblk : kThreads;
  const int R = kThreads / P;
  const int bpt = (nblk + P - 1) / P;
  const size_t total = (size_t)rows * nblk * kBlockBytes;
  int grid = (rows + R - 1) / R;
  if (grid > num_cus * 8) grid = num_cus * 8;
  for (int b0 = 0; b0 < batch;) {
    const int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    const float *xb = x + (size_t)b0 * cols;
    float *yb = y + (size_t)b0 * rows;
    if (nb == 4)
      q4_0_gemv_kernel<4><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, xb, yb, P, R, bpt);
    else if (nb == 2)
      q4_0_gemv_kernel<2><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, xb, yb, P, R, bpt);
    else
      q4_0_gemv_kernel<1><<<grid, kThreads, 0, s>>>(blocks, rows, cols, nblk, total, xb, yb, P, R, bpt);
    const hipError_t e = hipGetLastError();
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
