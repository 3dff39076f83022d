// Per-token symmetric int8 activations after the group FWHT.
//
// "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
// quantization", section 1: activations are 8-bit (W4A8) and each weight group
// is rotated by the orthogonal normalized Walsh-Hadamard matrix, so
// dot(w_g, x_g) = norm_g/G * dot(cb[idx_g], H_u x_g): the activation is
// rotated once here and the weights are never transformed back.
//
// One workgroup per token row, as many threads as the row has 8-element
// chunks (a multiple of 64, at most 1024).  Each lane owns 8 consecutive
// elements of a 128-wide group; 16 lanes hold one group.  Butterfly stages of
// half-width 1, 2, 4 are inside a lane, 8..64 across lanes (partner lane =
// lane ^ (h/8)), exchanged with DPP moves within each 16-lane row.
// Every stage computes (a+b, a-b) for the pair (j, j+h), j the lower index,
// in fp32, so the result is bit-identical to any fp32 evaluation of the same
// network.  Then s = max|u| / 127 over the row (1 for a zero row) and
// q = clip(rint(u / s), -127, 127), both divisions correctly rounded.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kPerLane = 8;
constexpr int kMaxChunksPerThread = 8;    // k <= 1024 * 8 * 8 = 65536

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}

// max over the wave (values are >= 0, so a 0 from an inactive DPP source is
// harmless); the result is valid in lanes 48..63.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<0x121, 0xF>(v));
  v = fmaxf(v, dpp_f<0x122, 0xF>(v));
  v = fmaxf(v, dpp_f<0x124, 0xF>(v));
  v = fmaxf(v, dpp_f<0x128, 0xF>(v));
  v = fmaxf(v, dpp_f<0x142, 0xA>(v));
  v = fmaxf(v, dpp_f<0x143, 0xC>(v));
  return v;
}

// The partner lane of the cross-lane stages (lane ^ 1, ^ 2, ^ 4, ^ 8 inside
// a 16-lane row), read with DPP: quad permutations for 1 and 2, the half-row
// mirror then the quad reversal for 4, a rotation by 8 within the row for 8.
template <int HL>
__device__ __forceinline__ float xor_lane(float v) {
  const int b = __builtin_bit_cast(int, v);
  if constexpr (HL == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));
  if constexpr (HL == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));
  if constexpr (HL == 4) {
    const int m = __builtin_amdgcn_mov_dpp(b, 0x141, 0xF, 0xF, true);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true));
  }
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true));
}

template <int HL, int CPT>
__device__ __forceinline__ void cross_stage(float (&v)[CPT][8], int c, int lane) {
  const bool upper = (lane & HL) != 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float other = xor_lane<HL>(v[c][e]);
    v[c][e] = upper ? (other - v[c][e]) : (v[c][e] + other);
  }
}

// u / s with IEEE round-to-nearest-even (HIP's default fp32 division is
// correctly rounded; spelled out so the intent survives compiler flags).
__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }

template <int CPT, int kThreads>
__global__ __launch_bounds__(kThreads) void act_fwht_quant_a8_kernel(
    const float *__restrict__ x, int k, int8_t *__restrict__ q, float *__restrict__ scale) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int chunks = k / kPerLane;           // 8-element chunks in the row
  const float *xr = x + (size_t)row * k;

  float v[CPT][kPerLane];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = t + c * kThreads;
    if (ci < chunks) {
      const float4 a = *reinterpret_cast<const float4 *>(xr + ci * kPerLane);
      const float4 b = *reinterpret_cast<const float4 *>(xr + ci * kPerLane + 4);
      v[c][0] = a.x; v[c][1] = a.y; v[c][2] = a.z; v[c][3] = a.w;
      v[c][4] = b.x; v[c][5] = b.y; v[c][6] = b.z; v[c][7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) v[c][e] = 0.0f;
    }
    // in-lane stages h = 1, 2, 4
#pragma unroll
    for (int h = 1; h < kPerLane; h <<= 1) {
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        if ((j & h) == 0) {
          const float a = v[c][j], b = v[c][j + h];
          v[c][j] = a + b;
          v[c][j + h] = a - b;
        }
      }
    }
    // cross-lane stages h = 8 .. 64: partner lane differs in bit (h/8) of lane%16.
    // Chunks with ci >= chunks belong to whole groups past the row end (k is a
    // multiple of 128 and 16 lanes hold one group), so their lanes exchange
    // only with each other.
    cross_stage<1>(v, c, lane);
    cross_stage<2>(v, c, lane);
    cross_stage<4>(v, c, lane);
    cross_stage<8>(v, c, lane);
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) amax = fmaxf(amax, fabsf(v[c][e]));
  }

  __shared__ float red[kThreads / kWave];
  __shared__ float s_shared;
  amax = wave_max_dpp(amax);
  if (lane == 63) red[t >> 6] = amax;
  __syncthreads();
  if (t == 0) {
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) m = fmaxf(m, red[w]);
    const float s = (m > 0.0f) ? div_rn(m, 127.0f) : 1.0f;
    s_shared = s;
    scale[row] = s;
  }
  __syncthreads();
  const float s = s_shared;

  int8_t *qr = q + (size_t)row * k;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = t + c * kThreads;
    if (ci < chunks) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        float r = rintf(div_rn(v[c][e], s));
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const uint32_t byte = (uint32_t)(uint8_t)(int8_t)(int)r;
        packed[e >> 2] |= byte << (8 * (e & 3));
      }
      *reinterpret_cast<uint2 *>(qr + ci * kPerLane) = make_uint2(packed[0], packed[1]);
    }
  }
}

// Group 1: the same per-token quantizer without the rotation (the transform
// of length 1 is the identity), for the Q4_0 products, whose weights carry no
// rotation.  k is any length (Q4_0 rows need not fill a 128-group): element i
// of the row belongs to thread i % kThreads.  s = max|x| / 127 (1 for a zero
// row), q = clip(rint(x / s), -127, 127), both divisions correctly rounded.
template <int EPT, int kThreads>
__global__ __launch_bounds__(kThreads) void act_quant_a8_unrotated_kernel(
    const float *__restrict__ x, int k, int8_t *__restrict__ q, float *__restrict__ scale) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const float *xr = x + (size_t)row * k;
  float v[EPT];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = t + e * kThreads;
    v[e] = i < k ? xr[i] : 0.0f;
    amax = fmaxf(amax, fabsf(v[e]));
  }
  __shared__ float red[kThreads / kWave];
  __shared__ float s_shared;
  amax = wave_max_dpp(amax);
  if ((t & 63) == 63) red[t >> 6] = amax;
  __syncthreads();
  if (t == 0) {
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) m = fmaxf(m, red[w]);
    const float s = (m > 0.0f) ? div_rn(m, 127.0f) : 1.0f;
    s_shared = s;
    scale[row] = s;
  }
  __syncthreads();
  const float s = s_shared;
  int8_t *qr = q + (size_t)row * k;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = t + e * kThreads;
    if (i < k) {
      const float r = fminf(fmaxf(rintf(div_rn(v[e], s)), -127.0f), 127.0f);
      qr[i] = (int8_t)(int)r;
    }
  }
}

}  // namespace

hipError_t launch_act_quant_a8_unrotated(const float *x, int m, int k, int8_t *q, float *scale,
                                         hipStream_t s) {
  const dim3 grid(m);
  if (k <= 256) act_quant_a8_unrotated_kernel<1, 256><<<grid, 256, 0, s>>>(x, k, q, scale);
  else if (k <= 1024) act_quant_a8_unrotated_kernel<1, 1024><<<grid, 1024, 0, s>>>(x, k, q, scale);
  else if (k <= 4096) act_quant_a8_unrotated_kernel<4, 1024><<<grid, 1024, 0, s>>>(x, k, q, scale);
  else if (k <= 16384) act_quant_a8_unrotated_kernel<16, 1024><<<grid, 1024, 0, s>>>(x, k, q, scale);
  else act_quant_a8_unrotated_kernel<64, 1024><<<grid, 1024, 0, s>>>(x, k, q, scale);   // k <= 65536
  return hipGetLastError();
}

hipError_t launch_act_fwht_quant_a8(const float *x, int m, int k, int8_t *q, float *scale,
                                    hipStream_t s) {
  const int chunks = k / kPerLane;               // a multiple of 16 (k % 128 == 0)
  const dim3 grid(m);
  // one chunk a thread up to 1024 chunks (threads rounded up to whole waves)
  if (chunks <= 64) act_fwht_quant_a8_kernel<1, 64><<<grid, 64, 0, s>>>(x, k, q, scale);
  else if (chunks <= 128) act_fwht_quant_a8_kernel<1, 128><<<grid, 128, 0, s>>>(x, k, q, scale);
  else if (chunks <= 256) act_fwht_quant_a8_kernel<1, 256><<<grid, 256, 0, s>>>(x, k, q, scale);
  else if (chunks <= 512) act_fwht_quant_a8_kernel<1, 512><<<grid, 512, 0, s>>>(x, k, q, scale);
  else if (chunks <= kMaxThreads)
    act_fwht_quant_a8_kernel<1, kMaxThreads><<<grid, kMaxThreads, 0, s>>>(x, k, q, scale);
  else if (chunks <= 2 * kMaxThreads)
    act_fwht_quant_a8_kernel<2, kMaxThreads><<<grid, kMaxThreads, 0, s>>>(x, k, q, scale);
  else if (chunks <= 4 * kMaxThreads)
    act_fwht_quant_a8_kernel<4, kMaxThreads><<<grid, kMaxThreads, 0, s>>>(x, k, q, scale);
  else
    act_fwht_quant_a8_kernel<kMaxChunksPerThread, kMaxThreads><<<grid, kMaxThreads, 0, s>>>(x, k, q, scale);
  return hipGetLastError();
}

}  // namespace bqm
