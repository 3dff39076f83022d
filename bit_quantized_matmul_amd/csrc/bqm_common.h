// Internal header shared by the libbqm HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bqm.h"

namespace bqm {

constexpr int kWave = 64;
constexpr int kGroup = 128;          // CQ quant group (the only one the device path builds)
constexpr int kTritsPerByte = 5;     // base-3 ternary: five indices a byte
constexpr int kTritBytes = (kGroup + kTritsPerByte - 1) / kTritsPerByte;   // 26 bytes a group
constexpr int kChunk = 32;           // indices a lane handles per load in the CQ kernels

// Level table handed to the CQ kernels by value.  For the fitted codebooks
// (bits 2/3/4) `h16`/`b16` hold the levels themselves as fp16 / bf16 bit
// patterns and `cscale` is 1.  For the analytic sets (bits 1, 5) they hold the
// signs -1/0/+1 and `cscale` is the set's level c, applied in fp32 at the end.
// Entries past the set's size (ternary field value 3) are 0.
struct LevelTable {
  uint16_t h16[16];
  uint16_t b16[16];
  float f32[16];    // fp32 levels (cb or c*sign), used by the encoder
  float cscale;
  int fold_exp;     // 13 - max(floor(log2(max |h16 level|)), -1): the GEMM's row exponent base
  int bits;         // bits code 1..6
  int index_bits;   // 1..4; 0 for base-3 ternary (five indices a byte)
  int levels;       // 2, 4, 8, 16 or 3
};

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// fp64 -> fp16 bit pattern, rounded once, half to even, for finite x >= 0 or
// negative x (sign kept).  Values that round past 65504 give +-inf (0x7C00).
__device__ __forceinline__ uint16_t f64_to_f16_rne_bits(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int e = (int)((b >> 52) & 0x7FF);
  uint64_t m = b & 0xFFFFFFFFFFFFFull;
  if (e == 0x7FF) return sign | 0x7C00u | (m ? 0x200u : 0u);
  if (e == 0) return sign;                          // fp64 subnormals are far below fp16's range
  int E = e - 1023 + 15;                            // fp16 biased exponent if normal
  uint64_t M = m | (1ull << 52);                    // 53-bit significand
  int shift = (E >= 1) ? 42 : 42 + (1 - E);         // keep 11 bits (normal) or fewer (subnormal)
  if (shift >= 64) return sign;                     // below half the smallest subnormal
  uint64_t kept = M >> shift;
  uint64_t rem = M & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  uint32_t h;
  if (E >= 1) {
    h = ((uint32_t)(E - 1) << 10) + (uint32_t)kept;  // kept carries the implicit bit; carry rolls E
    if (h >= 0x7C00u) h = 0x7C00u;
  } else {
    h = (uint32_t)kept;                             // subnormal; 1024 becomes the min normal
  }
  return sign | (uint16_t)h;
}

// fp64 -> nearest bfloat16 value (8 significant bits, half to even), as fp32.
// For finite normal inputs inside fp32's exponent range (the codebook levels).
__device__ __forceinline__ float f64_to_bf16_rne(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)((b >> 32) & 0x80000000u);
  int e = (int)((b >> 52) & 0x7FF);
  if (e == 0) return __uint_as_float(sign);
  uint64_t M = (b & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int shift = 45;                             // 53 -> 8 significant bits
  uint64_t kept = M >> shift;
  uint64_t rem = M & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  int E = e - 1023 + 127;                           // fp32 biased exponent
  uint32_t f = ((uint32_t)(E - 1) << 23) + ((uint32_t)kept << 16);
  return __uint_as_float(sign | f);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Wave-level sums / maxima over groups of `width` consecutive lanes (power of 2).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, WIDTH);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace bqm

// ------------------------------------------------------------ launch interfaces
// Each returns hipSuccess or the launch error.  Arguments are validated by the
// ABI layer (abi.hip) before these are called.
namespace bqm {

hipError_t launch_act_fwht_quant_a8(const float *x, int m, int k, int8_t *q, float *scale,
                                    hipStream_t s);
hipError_t launch_act_quant_a8_unrotated(const float *x, int m, int k, int8_t *q, float *scale,
                                         hipStream_t s);
hipError_t launch_q4_0_gemv_a8(const uint8_t *blocks, int rows, int cols, const int8_t *q,
                               const float *scale, int batch, float *y, hipStream_t s);
// Q4_0 A8 GEMV on fp32 activations, codes formed in the launch (batch <= 16;
// the supported predicate bounds the codes one workgroup holds in LDS).
bool q4_0_gemv_a8_fused_supported(int cols, int batch);
hipError_t launch_q4_0_gemv_a8_fused(const uint8_t *blocks, int rows, int cols, const float *x, int batch,
                                     float *y, int8_t *q_out, float *scale_out, int num_cus, hipStream_t s);
hipError_t launch_q4_0_gemm_a8(const uint8_t *blocks, int rows, int cols, const int8_t *q, const float *scale,
                               int m, float *y, int num_cus, hipStream_t s);
hipError_t launch_cq_gemv(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int batch, float *y,
                          int num_cus, hipStream_t s);
hipError_t launch_cq_gemv_f32(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                              const float *x, int batch, float *y, int8_t *q_out,
                              float *scale_out, int num_cus, hipStream_t s);
bool cq_gemv_mma_supported(const bqm_cq_layout &L, int batch);
// Base-3 packed ternary (bits code 6): one token with up to 128 groups a row,
// or 2..16 tokens (launches of up to 4) with up to 64.
bool cq_gemv_t3_supported(const bqm_cq_layout &L, int batch);
bool cq_t3_mma_supported(const bqm_cq_layout &L, int batch);
hipError_t launch_cq_t3_mma(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                            const int8_t *q, const float *scale, int batch, float *y, int num_cus,
                            hipStream_t s);
// Base-3 prefill GEMM: any m, any column count (group 128).
bool cq_t3_gemm_supported(const bqm_cq_layout &L, int m);
hipError_t launch_cq_t3_gemm(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                             const int8_t *q, const float *scale, int m, float *y, int num_cus,
                             hipStream_t s);
hipError_t launch_cq_gemv_t3(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                             const int8_t *q, const float *scale, int batch, float *y, int num_cus,
                             hipStream_t s);
bool cq_gemv_lut_supported(const bqm_cq_layout &L, int batch);
hipError_t launch_cq_gemv_lut(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T, const int8_t *q,
                              const float *scale, int batch, float *y, int num_cus, hipStream_t s);
hipError_t launch_cq_gemv_mma(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                              const int8_t *q, const float *scale, int batch, float *y,
                              int num_cus, hipStream_t s);
hipError_t launch_cq_gemm(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int m, float *y, int num_cus,
                          hipStream_t s);
hipError_t launch_q4_0_gemv(const uint8_t *blocks, int rows, int cols, const float *x, int batch,
                            float *y, int num_cus, hipStream_t s);
hipError_t launch_q4_0_gemm(const uint8_t *blocks, int rows, int cols, const float *x, int m,
                            float *y, int num_cus, hipStream_t s);
hipError_t launch_cq_pack(const float *w, const bqm_cq_layout &L, const LevelTable &T,
                          uint8_t *blob, int32_t *status, hipStream_t s);
hipError_t launch_q4_0_pack(const float *w, int rows, int cols, uint8_t *blocks, hipStream_t s);
hipError_t launch_codebook_fit(const double *samples, int64_t n, int levels, int iters,
                               double *raw, float *table, hipStream_t s);

}  // namespace bqm
