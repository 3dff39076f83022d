// CQ encoder: fp32 weights -> packed indices + fp16 group norms.
//
// "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
// quantization", section 1: each 128-wide group of an [out, in] row is
// rotated by the normalized Walsh-Hadamard transform; the rotated vector's
// direction is matched to the nearest entry of the Lloyd-Max codebook (only
// indices are kept) and its L2 norm is stored as fp16; indices are packed
// LSB-first, eight to a 64-bit word, low nibble = even column.
//
// Arithmetic (fp64, this file is built without FMA contraction), per group:
//   u = H_u w            butterfly, half-widths 1, 2, ..., 64, pair (j, j+h) -> (a+b, a-b)
//   ss = sum_i u_i*u_i   i ascending, product rounded, then added
//   r = sqrt(ss); norm = fp16_rne(r / sqrt(G)); t_i = u_i * (sqrt(G) / r), 0 if r == 0
//   idx_i = the first l minimizing |t_i - lv_l|      (lower index on a tie)
// The level scale reading: levels are on the N(0,1) scale, t = sqrt(G) y/||y||
// with y = H w (u/r = y/||y|| in real arithmetic).  sqrt and division are
// correctly rounded, so any implementation of this sequence gets the same bits.
//
// One wave per group: lane l holds u[l] and u[l+64]; stages h = 1..32 swap
// with lane l^h, stage 64 is inside the lane.  The norm sum runs on lane 0 in
// index order; lanes 0..15 then each pack one unit of 8 indices.
//
// Base-3 ternary (ib == 0, same levels and indices as the 2-bit ternary
// code): lanes 0..25 each write one byte, sum_i idx[5 lane + i] * 3^i, with
// digit 1 (the zero level) at the positions past the group's 128.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(b & 0xFFFFFFFFll), m, 64);
  const int hi = __shfl_xor((int)(b >> 32), m, 64);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__global__ __launch_bounds__(kThreads) void cq_pack_kernel(
    const float *__restrict__ w, int rows, int cols, int ib, uint8_t *__restrict__ blob,
    int64_t row_bytes, int64_t norms_offset, int64_t idx_bytes, int64_t total_bytes, LevelTable T,
    int32_t *__restrict__ status) {
  __shared__ double ubuf[kWaves][kGroup];
  __shared__ double ssbuf[kWaves];
  __shared__ uint8_t ibuf[kWaves][kGroup];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int ng = cols / kGroup;
  const long total = (long)rows * ng;
  uint16_t *norms = reinterpret_cast<uint16_t *>(blob + norms_offset);
  const double sqrt_g = __builtin_sqrt(128.0);

  // zero the padding bytes of the blob (at most 63 + 63 of them)
  if (blockIdx.x == 0) {
    for (int64_t o = idx_bytes + t; o < norms_offset; o += kThreads) blob[o] = 0;
    for (int64_t o = norms_offset + 2 * total + t; o < total_bytes; o += kThreads) blob[o] = 0;
  }

  for (long g0 = (long)blockIdx.x * kWaves; g0 < total; g0 += (long)gridDim.x * kWaves) {
    const long g = g0 + wave;
    const bool valid = g < total;
    const int row = valid ? (int)(g / ng) : 0;
    const int gi = valid ? (int)(g - (long)row * ng) : 0;
    double a = 0.0, b = 0.0;
    bool bad = false;
    if (valid) {
      const float *src = w + (size_t)row * cols + (size_t)gi * kGroup;
      const float fa = src[lane], fb = src[lane + 64];
      bad = !__builtin_isfinite(fa) || !__builtin_isfinite(fb);
      a = (double)fa;
      b = (double)fb;
    }
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      const double pa = shfl_xor_f64(a, h);
      const double pb = shfl_xor_f64(b, h);
      const bool upper = (lane & h) != 0;
      a = upper ? (pa - a) : (a + pa);
      b = upper ? (pb - b) : (b + pb);
    }
    {
      const double lo = a + b, hi = a - b;   // h = 64: pair (lane, lane + 64)
      a = lo;
      b = hi;
    }
    ubuf[wave][lane] = a;
    ubuf[wave][lane + 64] = b;
    __syncthreads();
    if (lane == 0) {
      double ss = 0.0;
      for (int i = 0; i < kGroup; ++i) {
        const double ui = ubuf[wave][i];
        const double sq = ui * ui;
        ss = ss + sq;
      }
      ssbuf[wave] = ss;
    }
    __syncthreads();
    const double ss = ssbuf[wave];
    const double r = __builtin_sqrt(ss);
    const double scale = (r > 0.0) ? (sqrt_g / r) : 0.0;
    const double ta = a * scale, tb = b * scale;
    int ia = 0, ibb = 0;
    double da = fabs(ta - (double)T.f32[0]), db = fabs(tb - (double)T.f32[0]);
    for (int l = 1; l < T.levels; ++l) {
      const double lv = (double)T.f32[l];
      const double xa = fabs(ta - lv), xb = fabs(tb - lv);
      if (xa < da) { da = xa; ia = l; }
      if (xb < db) { db = xb; ibb = l; }
    }
    ibuf[wave][lane] = (uint8_t)ia;
    ibuf[wave][lane + 64] = (uint8_t)ibb;
    __syncthreads();
    if (valid) {
      if (ib == 0) {
        if (lane < kTritBytes) {
          uint32_t v = 0;
#pragma unroll
          for (int i = kTritsPerByte - 1; i >= 0; --i) {
            const int p = kTritsPerByte * lane + i;
            v = 3u * v + (p < kGroup ? (uint32_t)ibuf[wave][p] : 1u);
          }
          blob[(int64_t)row * row_bytes + (int64_t)gi * kTritBytes + lane] = (uint8_t)v;
        }
      } else if (lane < 16) {
        uint64_t word = 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) word |= (uint64_t)ibuf[wave][8 * lane + s] << (ib * s);
        uint8_t *dst = blob + (int64_t)row * row_bytes + (int64_t)gi * 16 * ib + lane * ib;
        for (int k = 0; k < ib; ++k) dst[k] = (uint8_t)(word >> (8 * k));
      }
      if (lane == 0) {
        const double norm = r / sqrt_g;
        const uint16_t n16 = f64_to_f16_rne_bits(norm);
        norms[g] = n16;
        int32_t flags = 0;
        if ((n16 & 0x7C00u) == 0x7C00u) flags |= BQM_STATUS_NORM_OVERFLOW;
        if (flags && status) atomicOr(status, flags);
      }
      // any lane that saw a non-finite weight reports it
      if (bad && status) atomicOr(status, (int32_t)BQM_STATUS_NONFINITE);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_cq_pack(const float *w, const bqm_cq_layout &L, const LevelTable &T,
                          uint8_t *blob, int32_t *status, hipStream_t s) {
  const long total = (long)L.rows * (L.cols / kGroup);
  long grid = (total + kWaves - 1) / kWaves;
  if (grid > 16384) grid = 16384;
  if (grid < 1) grid = 1;
  cq_pack_kernel<<<(int)grid, kThreads, 0, s>>>(w, L.rows, L.cols, L.index_bits, blob,
                                                 L.idx_row_bytes, L.norms_offset, L.idx_bytes,
                                                 L.total_bytes, T, status);
  return hipGetLastError();
}

}  // namespace bqm
