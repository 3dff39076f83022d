// Prefill GEMM on packed CQ weights (matrix cores).
//
// "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
// quantization", section 3: prefill is a GEMM over the same pre-transposed
// [out, in] layout, each weight row one reduction stream; index and norm are
// unpacked in-stream with no transposed copy.  Section 1 fixes the group-128
// codebook + fp16-norm format.
//
//   Y[m, n] = scale[m] * cscale / 128 * sum_g norm[n, g] * sum_{k in g} q[m, k] * lv[idx[n, k]]
//
// This one is a dense contraction (M = 512 tokens: ~1000 flop per weight
// byte), so it runs on MFMA:
//  * A (activations): int8 q -> fp16 in LDS, exact (|q| <= 127), converted
//    with the 1024-bias trick: fp16 bits 0x6400 | (q + 128) equal 1152 + q.
//  * B (weights): each wave looks its own fragment up straight into registers
//    from an LDS table indexed by an index byte (the same replicated,
//    bank-conflict-free table as the GEMV).  Levels are bfloat16-representable
//    and so exact in fp16; with fp16 operands the products are exact and
//    the contraction accumulates in fp32 (v_mfma_f32_32x32x16_f16).
//  * Per group the MFMA chain starts from zero; the group's fp32 norm is then
//    applied per output column (acc += norm[n, g] * tile), so the norm never
//    rounds through a 16-bit operand.
//  * The k order inside a group is permuted consistently for A and B: in step
//    s (0..7) lane half h supplies columns 64h + 8s .. +8, so each lane reads
//    one contiguous run of 64 indices per group.
//  * Workgroup tiles are 128 (m) x 128 (n), 4 waves of 64 x 64.  Consecutive
//    tiles (the m-tiles of one n-block, which share weights) are mapped to the
//    same XCD: hardware deals workgroups round-robin over the 8 XCDs.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128, kBN = 128;
constexpr int kAStride = kGroup + 8;   // fp16 elements per A row in LDS (272 B: conflict-free b128 reads)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int IB> constexpr int table_rows() { return IB == 3 ? 64 : 256; }
template <int IB> constexpr int entry_bytes() { return IB == 1 ? 16 : (IB == 2 ? 8 : 4); }
template <int IB> constexpr int table_bytes() { return table_rows<IB>() * 256; }

template <int IB>
__device__ __forceinline__ uint4 table_entry16(int e, const LevelTable &T) {
  if constexpr (IB == 4 || IB == 3) {
    const int lo = (IB == 4) ? (e & 15) : (e & 7);
    const int hi = (IB == 4) ? (e >> 4) : (e >> 3);
    const uint32_t v = (uint32_t)T.h16[lo] | ((uint32_t)T.h16[hi] << 16);
    return make_uint4(v, v, v, v);
  } else if constexpr (IB == 2) {
    const uint32_t a = (uint32_t)T.h16[e & 3] | ((uint32_t)T.h16[(e >> 2) & 3] << 16);
    const uint32_t b = (uint32_t)T.h16[(e >> 4) & 3] | ((uint32_t)T.h16[(e >> 6) & 3] << 16);
    return make_uint4(a, b, a, b);
  } else {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = (uint32_t)T.h16[(e >> (2 * j)) & 1] | ((uint32_t)T.h16[(e >> (2 * j + 1)) & 1] << 16);
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
}

template <int K>
__device__ __forceinline__ uint32_t perm_addr(uint32_t w, uint32_t laneoff) {
  return __builtin_amdgcn_perm(w, laneoff, 0x0C0C0000u | ((4u + K) << 8));
}

// Bytes of indices a lane holds per group: 64 indices.
template <int IB> constexpr int lane_words() { return 2 * IB; }   // 8*IB bytes

// B operand for step s: the 8 levels of indices 8s..8s+7 of the lane's 64.
template <int IB>
__device__ __forceinline__ f16x8 lookup_step(const uint32_t (&wd)[2 * IB], int s,
                                             const uint8_t *tab, uint32_t laneoff) {
  uint32_t r[4];
  if constexpr (IB == 4) {           // one dword = 8 indices = 4 pair lookups
    const uint32_t w = wd[s];
    r[0] = *reinterpret_cast<const uint32_t *>(tab + perm_addr<0>(w, laneoff));
    r[1] = *reinterpret_cast<const uint32_t *>(tab + perm_addr<1>(w, laneoff));
    r[2] = *reinterpret_cast<const uint32_t *>(tab + perm_addr<2>(w, laneoff));
    r[3] = *reinterpret_cast<const uint32_t *>(tab + perm_addr<3>(w, laneoff));
  } else if constexpr (IB == 2) {    // two bytes -> two 4-level entries
    const uint32_t w = wd[s >> 1];
    uint2 e0, e1;
    if (s & 1) {
      e0 = *reinterpret_cast<const uint2 *>(tab + perm_addr<2>(w, laneoff));
      e1 = *reinterpret_cast<const uint2 *>(tab + perm_addr<3>(w, laneoff));
    } else {
      e0 = *reinterpret_cast<const uint2 *>(tab + perm_addr<0>(w, laneoff));
      e1 = *reinterpret_cast<const uint2 *>(tab + perm_addr<1>(w, laneoff));
    }
    r[0] = e0.x; r[1] = e0.y; r[2] = e1.x; r[3] = e1.y;
  } else if constexpr (IB == 1) {    // one byte -> one 8-level entry
    const uint32_t w = wd[s >> 2];
    uint4 e;
    switch (s & 3) {
      case 0: e = *reinterpret_cast<const uint4 *>(tab + perm_addr<0>(w, laneoff)); break;
      case 1: e = *reinterpret_cast<const uint4 *>(tab + perm_addr<1>(w, laneoff)); break;
      case 2: e = *reinterpret_cast<const uint4 *>(tab + perm_addr<2>(w, laneoff)); break;
      default: e = *reinterpret_cast<const uint4 *>(tab + perm_addr<3>(w, laneoff)); break;
    }
    r[0] = e.x; r[1] = e.y; r[2] = e.z; r[3] = e.w;
  } else {                           // IB == 3: 24 bits = four 6-bit pair fields
    const int bit = 24 * s;          // bit offset of the step's 8 indices
    const int wi = bit >> 5, sh = bit & 31;
    const uint32_t lo = wd[wi];
    const uint32_t hi = (wi + 1 < 2 * IB) ? wd[wi + 1] : 0u;
    const uint32_t v = __builtin_amdgcn_alignbit(hi, lo, sh);   // bits [bit, bit+32)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t f = (v >> (6 * p)) & 63u;
      r[p] = *reinterpret_cast<const uint32_t *>(tab + ((f << 8) | laneoff));
    }
  }
  f16x8 out;
  __builtin_memcpy(&out, r, 16);
  return out;
}

// int8 x4 (one dword) -> four fp16 values, exact: bits 0x6400 | (q + 128) = 1152 + q.
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
  const uint32_t u = w ^ 0x80808080u;                                // q + 128 per byte
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);   // [u0,0x64,u1,0x64]
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);   // [u2,0x64,u3,0x64]
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - bias);
}

template <int IB>
__global__ __launch_bounds__(kThreads) void cq_gemm_kernel(
    const uint8_t *__restrict__ idx, const uint16_t *__restrict__ norms,
    const int8_t *__restrict__ q, const float *__restrict__ scale, float *__restrict__ y,
    int M, int N, int K, int tiles_m, int tiles_n, LevelTable T) {
  constexpr int TB = table_bytes<IB>();
  __shared__ __align__(16) uint8_t tab[TB];
  __shared__ __align__(16) _Float16 As[2][kBM * kAStride];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  // XCD-aware tile order: tiles xcd*per .. xcd*per+per-1 run on one XCD
  const int ntiles = tiles_m * tiles_n;
  const int per = (ntiles + 7) / 8;
  const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (tile >= ntiles) return;
  const int mt = tile % tiles_m, nt = tile / tiles_m;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int ng = K / kGroup;
  const int row_bytes = K * IB / 8;
  const uint32_t laneoff = (uint32_t)(lane * entry_bytes<IB>()) & 255u;

  for (int o = t * 16; o < TB; o += kThreads * 16)
    *reinterpret_cast<uint4 *>(tab + o) = table_entry16<IB>(o >> 8, T);

  // A tile loader: thread t converts 64 int8 of row t/2, half t%2.
  const int arow = t >> 1, ahalf = t & 1;
  const bool arow_ok = (m0 + arow) < M;
  const int8_t *aptr = q + (size_t)(m0 + (arow_ok ? arow : 0)) * K + 64 * ahalf;
  uint4 apre[4];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      apre[i] = arow_ok ? *reinterpret_cast<const uint4 *>(aptr + (size_t)g * kGroup + 16 * i)
                        : make_uint4(0, 0, 0, 0);
  };
  auto store_a = [&](int buf) {
    _Float16 *dst = &As[buf][arow * kAStride + 64 * ahalf];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o[8];
      i8x4_to_f16x4(apre[i].x, o[0], o[1]);
      i8x4_to_f16x4(apre[i].y, o[2], o[3]);
      i8x4_to_f16x4(apre[i].z, o[4], o[5]);
      i8x4_to_f16x4(apre[i].w, o[6], o[7]);
      *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4 *>(dst + 16 * i + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  // B: per n-block nb, lane holds row n = n0 + 64 wn + 32 nb + lr, indices
  // 64 lh .. 64 lh + 63 of the current group.
  int ncol[2];
  bool nok[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    ncol[nb] = n0 + 64 * wn + 32 * nb + lr;
    nok[nb] = ncol[nb] < N;
  }
  uint32_t bw[2][2 * IB], bpre[2][2 * IB];
  uint16_t nrm16[2], nrmpre[2];
  auto load_b = [&](int g) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint8_t *p = idx + (size_t)(nok[nb] ? ncol[nb] : 0) * row_bytes +
                         (size_t)g * 16 * IB + 8 * IB * lh;
#pragma unroll
      for (int i = 0; i < 2 * IB; ++i)
        bpre[nb][i] = nok[nb] ? *reinterpret_cast<const uint32_t *>(p + 4 * i) : 0u;
      nrmpre[nb] = nok[nb] ? norms[(size_t)ncol[nb] * ng + g] : (uint16_t)0;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();

  for (int g = 0; g < ng; ++g) {
    const int buf = g & 1;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 2 * IB; ++i) bw[nb][i] = bpre[nb][i];
      nrm16[nb] = nrmpre[nb];
    }
    if (g + 1 < ng) {
      load_a(g + 1);
      load_b(g + 1);
    }
    f32x16 d[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) d[i][j][r] = 0.0f;
    const _Float16 *abase = &As[buf][(64 * wm + lr) * kAStride + 64 * lh];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      f16x8 a[2], b[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        a[mb] = *reinterpret_cast<const f16x8 *>(abase + 32 * mb * kAStride + 8 * s);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) b[nb] = lookup_step<IB>(bw[nb], s, tab, laneoff);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          d[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb], b[nb], d[mb][nb], 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float nv = half_bits_to_float(nrm16[nb]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][nb][r] = fmaf(nv, d[mb][nb][r], acc[mb][nb][r]);
    }
    if (g + 1 < ng) store_a(buf ^ 1);
    __syncthreads();
  }

  // epilogue: D row i = 8*(r/4) + 4*lh + (r%4), column lr
  const float cfac = T.cscale * (1.0f / kGroup);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 64 * wm + 32 * mb + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (m < M) {
        const float f = scale[m] * cfac;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          if (nok[nb]) y[(size_t)m * N + ncol[nb]] = acc[mb][nb][r] * f;
      }
    }
  }
}

}  // namespace

hipError_t launch_cq_gemm(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int m, float *y, int num_cus,
                          hipStream_t s) {
  (void)num_cus;
  const int tiles_m = (m + kBM - 1) / kBM;
  const int tiles_n = (L.rows + kBN - 1) / kBN;
  const int ntiles = tiles_m * tiles_n;
  const int grid = ((ntiles + 7) / 8) * 8;
  const uint16_t *norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  switch (L.index_bits) {
    case 1:
      cq_gemm_kernel<1><<<grid, kThreads, 0, s>>>(blob, norms, q, scale, y, m, L.rows, L.cols, tiles_m, tiles_n, T);
      break;
    case 2:
      cq_gemm_kernel<2><<<grid, kThreads, 0, s>>>(blob, norms, q, scale, y, m, L.rows, L.cols, tiles_m, tiles_n, T);
      break;
    case 3:
      cq_gemm_kernel<3><<<grid, kThreads, 0, s>>>(blob, norms, q, scale, y, m, L.rows, L.cols, tiles_m, tiles_n, T);
      break;
    default:
      cq_gemm_kernel<4><<<grid, kThreads, 0, s>>>(blob, norms, q, scale, y, m, L.rows, L.cols, tiles_m, tiles_n, T);
      break;
  }
  return hipGetLastError();
}

}  // namespace bqm
