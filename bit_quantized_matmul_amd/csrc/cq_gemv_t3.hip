// Decode GEMV on base-3 packed ternary CQ weights (bits code 6), 1..4 tokens a
// launch (several tokens: rows of at most 64 groups).
//
// Format: the ternary CQ set of the Needle .cact/W4A8 article (section 1;
// levels {-c, 0, +c}), with the indices packed five to a byte as base-3
// digits, the storage the llama.cpp TV-box / iPad page sets against 2-bit
// fields (its speed-up table, section 18).  Group of 128: 26 bytes, byte j = sum_i idx[5j+i] * 3^i, digit 1
// (the zero level) past the group's end.
//
// The rotated-domain identity (article, section 3) gives
//   y[b, n] = s_b * c / 128 * sum_g norm[n, g] * sum_{k in g} (idx[n, k] - 1) * q[b, k]
// and the inner sum is an exact integer (|.| <= 128 * 127), so it runs on
// v_dot4_i32_i8 with the digits as int8 -1 / 0 / +1.
//
// Layout of the work:
//  * A lane owns SL (1 or 2) group slots, groups li and li + P, for every row
//    it visits; a row takes P lanes (P a power of two, P * SL >= groups) and
//    a wave holds 64 / P rows at a time.  The lane's activations never change,
//    so they sit in registers for every token, rearranged once (read from a
//    copy of the tokens' codes that the workgroup stages in LDS, 144 bytes a
//    group so that
//    16 lanes reading 16 groups hit distinct banks): for weight byte j, the int8
//    codes at positions 5j .. 5j+3 as one dword, and the code at 5j+4 in
//    byte j % 4 of dword j / 4 of a second set (7 dwords a group).
//  * A weight byte's five digits come from an LDS table: entry v holds
//    digit_i(v) - 1 as int8 (i < 4 in the low dword, i = 4 in byte 0 of the
//    high dword), replicated 16 times with copy c at (16 v + c) * 8 bytes
//    (copy = lane % 16): two lanes of a half-wave share banks only when they
//    read different entries of equal parity, and the table (32 KB) is cheap
//    to build for every workgroup.
//  * A lane's 26 group bytes start 2-byte aligned: they come as the 32 bytes
//    from the 4-byte-aligned address below them, realigned with v_alignbyte.
//  * A wave walks at least two passes, the next pass's loads (the two
//    16-byte windows and the norm of each slot) in flight while one computes;
//    every load is unconditional (past the end: offset 0x80000000, zeros).
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kT3Threads = 512;                   // 8 waves share one table (2 blocks a CU)
constexpr int kT3Copies = 16;                      // table copies
constexpr int kT3Entries = 256;                    // every byte value (243.. are not digits: zeros)
constexpr int kT3TableBytes = kT3Entries * kT3Copies * 8;   // 32 KB
constexpr uint32_t kT3OOB = 0x80000000u;
constexpr int kT3MaxGroups = 128;                  // cols <= 16384 (one token)
constexpr int kT3MaxGroupsBatched = 64;            // cols <= 8192 (several tokens)
constexpr int kT3QStride = kGroup + 16;            // bytes a group in the LDS copy of the codes
typedef uint32_t u32x4t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_t3(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// One slot's inputs for one row: 32 bytes of weights from the aligned
// address below the group, and the dword holding its fp16 norm.
struct T3Load {
  uint32_t w[8];
  uint32_t nw;
};

template <int SL, int BATCH>
__global__ __launch_bounds__(kT3Threads) void cq_gemv_t3_kernel(
    const uint8_t *__restrict__ idx, uint32_t blob_bytes, const uint16_t *__restrict__ norms,
    uint32_t norm_bytes, const int8_t *__restrict__ q, const float *__restrict__ scale,
    float *__restrict__ y, int rows, int ng, int plog2, int passes_per_wave, float cfac) {
  __shared__ __align__(16) uint8_t tab[kT3TableBytes];
  extern __shared__ __align__(16) uint8_t qlds[];   // [BATCH][ng][kT3QStride]
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int P = 1 << plog2;
  const int li = lane & (P - 1);
  const int rr = lane >> plog2;                    // row within a pass
  const int rpp = 64 >> plog2;                     // rows per pass
  const uint32_t row_bytes = (uint32_t)ng * kTritBytes;

  // the digit table: entry v, copy c at (32 v + c) * 8 (byte values past
  // 242 are no base-3 digits: zero rows, so any byte addresses the table).
  // Thread t computes entry t % 256 once and writes half of its copies, two
  // to a 16-byte store.
  {
    static_assert(kT3Threads == 2 * kT3Entries, "two threads per table entry");
    const uint32_t v0 = (uint32_t)t & (kT3Entries - 1);
    uint32_t v = v0, d[kTritsPerByte];
#pragma unroll
    for (int i = 0; i < kTritsPerByte; ++i) {
      d[i] = (v % 3u + 0xFFu) & 0xFFu;             // digit - 1 as an int8 bit pattern
      v /= 3u;
    }
    const uint32_t lo = v0 < 243u ? (d[0] | (d[1] << 8) | (d[2] << 16) | (d[3] << 24)) : 0u;
    const uint32_t hi = v0 < 243u ? d[4] : 0u;
    uint4 *row = reinterpret_cast<uint4 *>(tab + (size_t)v0 * kT3Copies * 8) + (t >> 8) * (kT3Copies / 4);
#pragma unroll
    for (int c = 0; c < kT3Copies / 4; ++c) row[c] = make_uint4(lo, hi, lo, hi);
  }

  // the tokens' codes into LDS, 16 bytes a thread per step
  for (int c = t; c < BATCH * ng * (kGroup / 16); c += kT3Threads) {
    const int g = c >> 3, w = c & 7;               // g: token * ng + group (q is [BATCH][cols])
    *reinterpret_cast<u32x4t *>(qlds + g * kT3QStride + 16 * w) =
        *reinterpret_cast<const u32x4t *>(q + (size_t)c * 16);
  }
  __syncthreads();

  // the lane's activations per slot, five positions per weight byte
  constexpr int kQB = (kTritBytes + 3) / 4;
  uint32_t qa[SL][BATCH][kTritBytes], qb[SL][BATCH][kQB];
#pragma unroll
  for (int s = 0; s < SL; ++s)
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    const int g = li + P * s;
    uint32_t qw[kGroup / 4 + 1];
    if (g < ng) {
      const u32x4t *src = reinterpret_cast<const u32x4t *>(qlds + (b * ng + g) * kT3QStride);
#pragma unroll
      for (int i = 0; i < kGroup / 16; ++i) {
        const u32x4t v = src[i];
        qw[4 * i] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kGroup / 4; ++i) qw[i] = 0u;
    }
    qw[kGroup / 4] = 0u;                           // positions 128.. read as 0 (their digits are 1)
#pragma unroll
    for (int i = 0; i < kQB; ++i) qb[s][b][i] = 0u;
#pragma unroll
    for (int j = 0; j < kTritBytes; ++j) {
      const int p = kTritsPerByte * j;             // positions p .. p + 4
      qa[s][b][j] = __builtin_amdgcn_alignbyte(qw[(p >> 2) + 1], qw[p >> 2], p & 3);
      const int p4 = p + 4;
      qb[s][b][j >> 2] |= ((qw[p4 >> 2] >> (8 * (p4 & 3))) & 0xFFu) << (8 * (j & 3));
    }
  }

  // the whole blob: a group's 32-byte window can reach 6 bytes past the
  // indices, into the padding and norms that follow them
  const __amdgpu_buffer_rsrc_t rw = rsrc_t3(idx, blob_bytes);
  const __amdgpu_buffer_rsrc_t rn = rsrc_t3(norms, norm_bytes);
  const uint32_t copyoff = (uint32_t)(lane & (kT3Copies - 1)) * 8u;
  const int wave_g = (int)((blockIdx.x * kT3Threads + t) >> 6);
  const int pass0 = wave_g * passes_per_wave;
  float sfac[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) sfac[b] = scale[b] * cfac;

  // byte offset of slot s of row n (or past every range)
  auto woff = [&](int n, int s) -> uint32_t {
    const int g = li + P * s;
    return (n < rows && g < ng) ? (uint32_t)n * row_bytes + (uint32_t)g * kTritBytes : kT3OOB;
  };
  auto noff = [&](int n, int s) -> uint32_t {
    const int g = li + P * s;
    return (n < rows && g < ng) ? ((uint32_t)n * (uint32_t)ng + (uint32_t)g) * 2u : kT3OOB;
  };
  auto row_of = [&](int pass) { return pass * rpp + rr; };
  auto issue = [&](T3Load (&L)[SL], int pass) {
    const int n = pass < pass0 + passes_per_wave ? row_of(pass) : rows;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint32_t o = woff(n, s);
      const uint32_t a = o == kT3OOB ? kT3OOB : (o & ~3u);
      const u32x4t v0 = __builtin_bit_cast(u32x4t, __builtin_amdgcn_raw_buffer_load_b128(rw, a, 0, 0));
      const u32x4t v1 = __builtin_bit_cast(u32x4t, __builtin_amdgcn_raw_buffer_load_b128(rw, a + 16u, 0, 0));
      L[s].w[0] = v0.x; L[s].w[1] = v0.y; L[s].w[2] = v0.z; L[s].w[3] = v0.w;
      L[s].w[4] = v1.x; L[s].w[5] = v1.y; L[s].w[6] = v1.z; L[s].w[7] = v1.w;
      const uint32_t no = noff(n, s);
      L[s].nw = __builtin_amdgcn_raw_buffer_load_b32(rn, no == kT3OOB ? kT3OOB : (no & ~3u), 0, 0);
    }
  };
  auto compute = [&](T3Load (&L)[SL], int pass) {
    const int n = row_of(pass);
    float part[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) part[b] = 0.0f;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint32_t o = woff(n, s);
      const uint32_t sh = o & 3u;                  // 0 or 2
      uint32_t r[7];
#pragma unroll
      for (int i = 0; i < 7; ++i) r[i] = __builtin_amdgcn_alignbyte(L[s].w[i + 1], L[s].w[i], sh);
      int acc[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) acc[b] = 0;
#pragma unroll
      for (int j = 0; j < kTritBytes; ++j) {
        const uint32_t addr = ((r[j >> 2] >> (8 * (j & 3))) & 0xFFu) * (kT3Copies * 8u) + copyoff;
        const uint2 e = *reinterpret_cast<const uint2 *>(tab + addr);
        // the fifth digit moves to byte j % 4, where its code sits
        const uint32_t e5 = e.y << (8 * (j & 3));
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          acc[b] = __builtin_amdgcn_sdot4((int)e.x, (int)qa[s][b][j], acc[b], false);
          acc[b] = __builtin_amdgcn_sdot4((int)e5, (int)qb[s][b][j >> 2], acc[b], false);
        }
      }
      const uint32_t no = noff(n, s);
      const float nrm = half_bits_to_float((uint16_t)(L[s].nw >> ((no & 2u) * 8u)));
#pragma unroll
      for (int b = 0; b < BATCH; ++b) part[b] += (float)acc[b] * nrm;   // 0 past the row (acc = 0)
    }
    // the row's P lanes add their parts (xor steps stay inside the segment)
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      for (int m = P >> 1; m > 0; m >>= 1) part[b] += __shfl_xor(part[b], m, 64);
    if (li == 0 && n < rows && pass < pass0 + passes_per_wave) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) y[(size_t)b * rows + n] = part[b] * sfac[b];
    }
  };

  T3Load A[SL], Bq[SL];
  issue(A, pass0);
  for (int p = pass0; p < pass0 + passes_per_wave; p += 2) {
    issue(Bq, p + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, p);
    __builtin_amdgcn_sched_barrier(0);
    if (p + 1 < pass0 + passes_per_wave) {        // uniform
      issue(A, p + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(Bq, p + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace

bool cq_gemv_t3_supported(const bqm_cq_layout &L, int batch) {
  const int ng = L.cols / kGroup;
  const int max_groups = batch == 1 ? kT3MaxGroups : kT3MaxGroupsBatched;
  return batch >= 1 && batch <= 16 && L.group == kGroup && L.cols % kGroup == 0 && ng >= 1 &&
         (ng <= max_groups || cq_t3_mma_supported(L, batch)) && L.total_bytes < ((int64_t)1 << 31);
}

namespace {

template <int SL, int BATCH>
hipError_t launch_t3(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T, const int8_t *q,
                     const float *scale, float *y, int num_cus, hipStream_t s) {
  const int ng = L.cols / kGroup;
  const int need = (ng + SL - 1) / SL;             // lanes per row
  int plog2 = 0;
  while ((1 << plog2) < need) ++plog2;
  const int rpp = 64 >> plog2;
  const long passes = ((long)L.rows + rpp - 1) / rpp;
  // resident workgroups a CU: two, one when several tokens' codes in
  // registers leave room for only two waves a SIMD
  const long waves_max = (long)num_cus * (BATCH > 1 ? 1 : 2) * (kT3Threads / kWave);
  // at least 2 passes a wave (its activation set-up is not repeated per row),
  // as many waves as that gives up to the resident workgroups
  const long waves = (passes + 1) / 2 < waves_max ? (passes + 1) / 2 : waves_max;
  const int per_wave = (int)((passes + waves - 1) / waves);
  const long used = (passes + per_wave - 1) / per_wave;          // waves with work
  const int blocks = (int)((used + (kT3Threads / kWave) - 1) / (kT3Threads / kWave));
  const uint16_t *norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  const uint32_t nb = (uint32_t)((L.norms_count * 2 + 3) & ~(int64_t)3);
  const size_t lds = (size_t)BATCH * ng * kT3QStride;   // the tokens' codes (the table is static)
  cq_gemv_t3_kernel<SL, BATCH><<<blocks, kT3Threads, lds, s>>>(blob, (uint32_t)L.total_bytes, norms, nb, q,
                                                               scale, y, L.rows, ng, plog2, per_wave,
                                                               T.cscale / (float)kGroup);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cq_gemv_t3(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                             const int8_t *q, const float *scale, int batch, float *y, int num_cus,
                             hipStream_t s) {
  if (batch == 1)
    return L.cols / kGroup > 64 ? launch_t3<2, 1>(blob, L, T, q, scale, y, num_cus, s)
                                : launch_t3<1, 1>(blob, L, T, q, scale, y, num_cus, s);
  // several tokens: one pass over the weights on the int8 matrix cores
  if (cq_t3_mma_supported(L, batch)) return launch_cq_t3_mma(blob, L, T, q, scale, batch, y, num_cus, s);
  // (rows of at most 64 groups) launches of 4, 2 and 1 tokens, each one pass
  // over the weights
  for (int b0 = 0; b0 < batch;) {
    const int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    const int8_t *qb = q + (size_t)b0 * L.cols;
    float *yb = y + (size_t)b0 * L.rows;
    hipError_t e;
    if (nb == 4) e = launch_t3<1, 4>(blob, L, T, qb, scale + b0, yb, num_cus, s);
    else if (nb == 2) e = launch_t3<1, 2>(blob, L, T, qb, scale + b0, yb, num_cus, s);
    else e = launch_t3<1, 1>(blob, L, T, qb, scale + b0, yb, num_cus, s);
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

}  // namespace bqm
