// Lookup-table decode GEMV for binary and ternary CQ weights.
//
// "llama.cpp on a TV box and a 2013 iPad Air" (smolmaxxing), the kernel
// table's entry on the 1-bit LUT kernel: instead of decoding each weight, a
// table of the partial sums of a few activations over every sign pattern is
// built once, and each group of weight bits then costs one table lookup (the
// Four-Russians / T-MAC method).  The CQ sum it computes is the GEMV's
// (Needle article, section 1: the analytic binary / ternary sets, levels
// c * sign):
//   y[b, n] = scale[b] * c / 128 * sum_g norm[n, g] * sum_{i in g} sign(idx[n, i]) * q[b, i]
//
// Tables: binary weights are one bit each (1 = +, 0 = -), so a nibble of the
// index stream covers 4 activations and the table of activations 4u .. 4u+3
// holds T_u[e] = sum_t (bit t of e ? +q : -q)[4u + t] for e = 0..15.
// Ternary weights are 2-bit fields (0 = -, 1 = 0, 2 = +, 3 = 0), so a nibble
// covers 2 activations and T_u[e] = lv(e & 3) q[2u] + lv(e >> 2) q[2u + 1].
// Entries are int16 (|T| <= 4 * 127) with the BATCH tokens side by side, so
// one LDS read returns every token's partial sum and one packed int16 add
// accumulates two tokens.  A group's sums are then widened, scaled by its
// fp32 norm, and the row's groups are added in fp32 across lanes in a fixed
// order.  All integer sums are exact.
//
// Work: one 512-thread workgroup per CU builds the tables for all columns,
// then its waves walk its rows: a lane owns one 128-wide group of a row (16
// or 32 index bytes and the norm), P lanes share a row, and four steps of
// loads are in flight.  A group sums at most 32 (binary) or 64 (ternary)
// entries, |sum| <= 16256: within int16.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kLutThreads = 512;
constexpr int kLutWaves = kLutThreads / kWave;
constexpr int kLutMaxGroups = 64;                   // a lane per group: cols <= 8192
constexpr uint32_t kLutOOB = 0x80000000u;
constexpr size_t kLutMaxTable = 128 * 1024;         // LDS for the tables
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t lut_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// TER: ternary 2-bit fields (else binary bits).  BATCH: tokens side by side
// in an entry (1, 2 or 4); nb <= BATCH of them are real.
template <bool TER, int BATCH>
__global__ __launch_bounds__(kLutThreads) void cq_gemv_lut_kernel(
    const uint8_t *__restrict__ idx, const uint16_t *__restrict__ norms, const int8_t *__restrict__ q,
    const float *__restrict__ scale, float *__restrict__ y, int rows, int cols, int nb, int rows_per_block,
    int plog2, uint32_t idx_bytes, uint32_t norm_bytes, float cfac) {
  constexpr int kPer = TER ? 2 : 4;                 // activations a table covers
  extern __shared__ __align__(16) uint16_t tab[];   // [unit][16 entries][BATCH] int16
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int units = cols / kPer;
  const int ng = cols / kGroup;

  // ---- 1. the tables
  for (int u = t; u < units; u += kLutThreads) {
    int a[BATCH][kPer];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
#pragma unroll
      for (int k = 0; k < kPer; ++k) a[b][k] = b < nb ? (int)q[(size_t)b * cols + kPer * u + k] : 0;
    uint16_t ent[16][BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if constexpr (TER) {
        const int l0[4] = {-a[b][0], 0, a[b][0], 0};
        const int l1[4] = {-a[b][1], 0, a[b][1], 0};
#pragma unroll
        for (int e = 0; e < 16; ++e) ent[e][b] = (uint16_t)(short)(l0[e & 3] + l1[e >> 2]);
      } else {
        int lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = ((e & 1) ? a[b][0] : -a[b][0]) + ((e & 2) ? a[b][1] : -a[b][1]);
          hi[e] = ((e & 1) ? a[b][2] : -a[b][2]) + ((e & 2) ? a[b][3] : -a[b][3]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) ent[e][b] = (uint16_t)(short)(lo[e & 3] + hi[e >> 2]);
      }
    }
    // 16 x BATCH halfwords = 2 x BATCH 16-byte stores
    uint32_t w[8 * BATCH];
#pragma unroll
    for (int i = 0; i < 8 * BATCH; ++i) {
      const int h0 = 2 * i, h1 = 2 * i + 1;        // halfword index e * BATCH + b
      w[i] = (uint32_t)ent[h0 / BATCH][h0 % BATCH] | ((uint32_t)ent[h1 / BATCH][h1 % BATCH] << 16);
    }
#pragma unroll
    for (int i = 0; i < 2 * BATCH; ++i)
      *reinterpret_cast<uint4 *>(&tab[(size_t)u * 16 * BATCH + 8 * i]) = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  }
  __syncthreads();

  // ---- 2. rows: a lane owns one 128-wide group of a row (the group's index
  // bytes in one or two 16-byte loads, and its norm); P lanes (the power of
  // two covering the groups) share a row, so a wave step covers 64 / P rows
  // of the workgroup's run; kLutDepth steps of loads are in flight.
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(rows, r0 + rows_per_block);
  const __amdgpu_buffer_rsrc_t ri = lut_rsrc(idx, idx_bytes);
  const __amdgpu_buffer_rsrc_t rn = lut_rsrc(norms, norm_bytes);
  constexpr int kGB = TER ? 32 : 16;                // index bytes of a group
  constexpr int kGW = kGB / 4;                      // their dwords
  constexpr int kGN = 2 * kGB;                      // nibbles (lookups) of a group
  const int P = 1 << plog2;
  const int g = lane & (P - 1);                     // the lane's group
  const int rs = lane >> plog2;                     // its row within the step
  const int rps = (kWave >> plog2) * kLutWaves;     // rows a workgroup step covers
  const int row_bytes = ng * kGB;
  auto load = [&](int step, uint32_t (&wd)[kGW], uint32_t &nw) {
    const int row = r0 + step * rps + wave * (kWave >> plog2) + rs;
    const bool ok = row < r1 && g < ng;
    const uint32_t o = ok ? (uint32_t)row * (uint32_t)row_bytes + (uint32_t)g * kGB : kLutOOB;
#pragma unroll
    for (int h = 0; h < kGW / 4; ++h) {
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ri, o + 16u * h, 0, 0));
      wd[4 * h] = v.x; wd[4 * h + 1] = v.y; wd[4 * h + 2] = v.z; wd[4 * h + 3] = v.w;
    }
    const uint32_t no = ok ? ((uint32_t)row * (uint32_t)ng + (uint32_t)g) * 2u : kLutOOB;
    nw = __builtin_amdgcn_raw_buffer_load_b32(rn, no & ~3u, 0, 0) >> ((no & 2u) * 8u);
  };
  constexpr int kLutDepth = 4;
  uint32_t ring[kLutDepth][kGW], nring[kLutDepth];
  const int steps = (r1 - r0 + rps - 1) / rps;
#pragma unroll
  for (int d = 0; d < kLutDepth; ++d) load(d, ring[d], nring[d]);
  const uint8_t *tb = reinterpret_cast<const uint8_t *>(tab);
  // the group's first table (lanes past the row's groups read table 0, with
  // a zero norm, so that no address leaves the tables)
  const uint32_t ubase = (uint32_t)(g < ng ? g : 0) * kGN;
  for (int s0 = 0; s0 < steps; s0 += kLutDepth) {
#pragma unroll
    for (int d = 0; d < kLutDepth; ++d) {
      const int step = s0 + d;
      float acc[BATCH];
      s16x2 s2[(BATCH + 1) / 2];
      int s1 = 0;
#pragma unroll
      for (int i = 0; i < (BATCH + 1) / 2; ++i) s2[i] = s16x2{0, 0};
#pragma unroll
      for (int p = 0; p < kGN; ++p) {
        const uint32_t nib = (ring[d][p >> 3] >> (4 * (p & 7))) & 15u;
        const uint32_t a = ((ubase + p) * 16u + nib) * (2u * BATCH);   // byte address of the entry
        if constexpr (BATCH == 1) {
          s1 += (int)*reinterpret_cast<const short *>(tb + a);
        } else if constexpr (BATCH == 2) {
          s2[0] += *reinterpret_cast<const s16x2 *>(tb + a);
        } else {
          const uint2 e = *reinterpret_cast<const uint2 *>(tb + a);
          s2[0] += __builtin_bit_cast(s16x2, e.x);
          s2[1] += __builtin_bit_cast(s16x2, e.y);
        }
      }
      // lanes without a group (or past the rows) read zero words and a zero
      // norm: their sums are multiplied by 0
      const float nv = half_bits_to_float((uint16_t)nring[d]);
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        acc[b] = nv * (BATCH == 1 ? (float)s1 : (float)s2[b >> 1][b & 1]);
      load(step + kLutDepth, ring[d], nring[d]);   // refill: kLutDepth steps ahead
      // the row's groups meet across its P lanes (a fixed order)
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        for (int o = P >> 1; o >= 1; o >>= 1) acc[b] += __shfl_xor(acc[b], o, 64);
      const int row = r0 + step * rps + wave * (kWave >> plog2) + rs;
      if (step < steps && g == 0 && row < r1) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
          if (b < nb) y[(size_t)b * rows + row] = acc[b] * (scale[b] * cfac);
      }
    }
  }
}

size_t lut_table_bytes(bool ter, int cols, int batch) {
  return (size_t)(cols / (ter ? 2 : 4)) * 16 * 2 * batch;
}

}  // namespace

bool cq_gemv_lut_supported(const bqm_cq_layout &L, int batch) {
  const bool ter = L.bits == BQM_CQ_TERNARY;
  if ((L.bits != BQM_CQ_BINARY && !ter) || batch < 1 || batch > 16 || L.cols % kGroup) return false;
  if (L.cols / kGroup > kLutMaxGroups) return false;
  if (lut_table_bytes(ter, L.cols, 1) > kLutMaxTable) return false;
  return (uint64_t)L.idx_bytes < (1u << 31) && (uint64_t)L.norms_count * 2 < (1u << 31);
}

hipError_t launch_cq_gemv_lut(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T, const int8_t *q,
                              const float *scale, int batch, float *y, int num_cus, hipStream_t s) {
  const bool ter = L.bits == BQM_CQ_TERNARY;
  const int ng = L.cols / kGroup;
  int plog2 = 0;
  while ((1 << plog2) < ng) ++plog2;
  const int rps = (kWave >> plog2) * kLutWaves;    // rows a workgroup step covers
  int blocks = (L.rows + rps - 1) / rps;
  if (blocks > num_cus) blocks = num_cus;
  const int rpb = (L.rows + blocks - 1) / blocks;
  blocks = (L.rows + rpb - 1) / rpb;
  const uint16_t *norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  const uint32_t nbytes = (uint32_t)((L.norms_count * 2 + 3) & ~(int64_t)3);
  const float cfac = T.cscale * (1.0f / kGroup);
  for (int b0 = 0; b0 < batch;) {
    // tokens side by side: 4 for 3 or 4 left (the fourth entry of 3 holds
    // zeros), 2 for 2, 1 for 1; fewer while the tables would not fit
    const int left = batch - b0;
    int bt = left >= 3 ? 4 : (left == 2 ? 2 : 1);
    while (bt > 1 && lut_table_bytes(ter, L.cols, bt) > kLutMaxTable) bt >>= 1;
    const int nb = left < bt ? left : bt;
    const size_t lds = lut_table_bytes(ter, L.cols, bt);
    const int8_t *qb = q + (size_t)b0 * L.cols;
    float *yb = y + (size_t)b0 * L.rows;
    const float *sb = scale + b0;
#define BQM_LUT_GO(TT, BB)                                                                          \
  cq_gemv_lut_kernel<TT, BB><<<blocks, kLutThreads, lds, s>>>(blob, norms, qb, sb, yb, L.rows, L.cols, nb, \
                                                             rpb, plog2, (uint32_t)L.idx_bytes, nbytes, cfac)
    if (ter) {
      if (bt == 4) BQM_LUT_GO(true, 4); else if (bt == 2) BQM_LUT_GO(true, 2); else BQM_LUT_GO(true, 1);
    } else {
      if (bt == 4) BQM_LUT_GO(false, 4); else if (bt == 2) BQM_LUT_GO(false, 2); else BQM_LUT_GO(false, 1);
    }
#undef BQM_LUT_GO
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

}  // namespace bqm
