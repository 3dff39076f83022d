// Decode GEMV on packed CQ weights.
//
// "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
// quantization": section 1 defines the format (group-128 Walsh-Hadamard
// rotation, indices into a shared Lloyd-Max codebook, fp16 group norm,
// LSB-first index packing); section 3 says decode is a GEMV that streams the
// pre-transposed [out, in] rows and unpacks index and norm in-stream.  The
// companion mmap article adds that dequantization happens in the kernel.
//
// The sum computed, per output row n and token b (rotated domain, so the
// weights are never inverse-transformed):
//   y[b, n] = scale[b] * cscale / 128 * sum_g norm[n, g] * sum_{i in g} lv[idx[n, i]] * q[b, i]
//
// Design (MI355X):
//  * The kernel is HBM-bound: every byte of indices and norms is read once,
//    with each wave instruction covering 64 lanes x 4*bits contiguous bytes
//    (dwordx4 for 4-bit).  A lane always handles the same 32-index chunks of
//    a row, so its activations sit in registers as fp16 pairs for the whole
//    kernel.
//  * Index -> level lookup goes through an LDS table keyed by one index byte:
//    4-bit -> 2 fp16 levels, 2-bit -> 4, 1-bit -> 8; 3-bit uses 6-bit fields
//    (2 levels).  Each table row is 256 bytes holding copies of the entry at
//    lane-specific offsets, so a wave's lookups never conflict on a bank, and
//    one v_perm_b32 forms the address (index byte << 8) | lane offset.
//  * Products run on v_dot2_f32_f16 (fp16 x fp16 exact, fp32 accumulate).
//    The codebook levels are bfloat16-representable, hence exact in fp16, and
//    |q| <= 127 is exact in fp16.
//  * Row sums reduce across the lanes that share a row with xor shuffles,
//    then across waves (when a row is split over several waves) through LDS
//    in a fixed order, so results are deterministic.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesPerBlock = kThreads / kWave;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int IB>
struct Chunk;   // raw index bytes of one 32-index chunk
template <> struct Chunk<1> { uint32_t w[1]; };
template <> struct Chunk<2> { uint32_t w[2]; };
template <> struct Chunk<3> { uint32_t w[3]; };
template <> struct Chunk<4> { uint32_t w[4]; };

template <int IB>
__device__ __forceinline__ Chunk<IB> load_chunk(const uint8_t *p) {
  Chunk<IB> c;
  if constexpr (IB == 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else if constexpr (IB == 3) {
    const uint32_t *u = reinterpret_cast<const uint32_t *>(p);
    c.w[0] = __builtin_nontemporal_load(u);
    c.w[1] = __builtin_nontemporal_load(u + 1);
    c.w[2] = __builtin_nontemporal_load(u + 2);
  } else if constexpr (IB == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    c.w[0] = v.x; c.w[1] = v.y;
  } else {
    c.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
  }
  return c;
}

// Table bytes and entry size per index width.
template <int IB> constexpr int table_rows() { return IB == 3 ? 64 : 256; }
template <int IB> constexpr int entry_bytes() { return IB == 1 ? 16 : (IB == 2 ? 8 : 4); }
template <int IB> constexpr int table_bytes() { return table_rows<IB>() * 256; }

// Levels (fp16 bits) of table row `e`, packed as the row's entry.
template <int IB>
__device__ __forceinline__ uint4 table_entry16(int e, const LevelTable &T) {
  // returns 16 bytes = the entry replicated to fill 16 bytes
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

// LDS address of index byte `byte_sel` of word w: (byte << 8) | lane offset.
// v_perm_b32 picks result byte 0 from `laneoff` byte 0 (selector 0) and result
// byte 1 from w's byte k (selector 4+k); selector 0x0C yields zero bytes.
template <int K>
__device__ __forceinline__ uint32_t perm_addr(uint32_t w, uint32_t laneoff) {
  return __builtin_amdgcn_perm(w, laneoff, 0x0C0C0000u | ((4u + K) << 8));
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t *smem, uint32_t a) {
  return *reinterpret_cast<const uint32_t *>(smem + a);
}
__device__ __forceinline__ uint2 lds_u64(const uint8_t *smem, uint32_t a) {
  return *reinterpret_cast<const uint2 *>(smem + a);
}
__device__ __forceinline__ uint4 lds_u128(const uint8_t *smem, uint32_t a) {
  return *reinterpret_cast<const uint4 *>(smem + a);
}

// Look up the 16 fp16 level pairs (pair j = indices 2j, 2j+1) of one chunk.
template <int IB>
__device__ __forceinline__ void lookup(const Chunk<IB> &c, const uint8_t *smem, uint32_t laneoff,
                                       uint32_t W[16]) {
  if constexpr (IB == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      W[4 * d + 0] = lds_u32(smem, perm_addr<0>(c.w[d], laneoff));
      W[4 * d + 1] = lds_u32(smem, perm_addr<1>(c.w[d], laneoff));
      W[4 * d + 2] = lds_u32(smem, perm_addr<2>(c.w[d], laneoff));
      W[4 * d + 3] = lds_u32(smem, perm_addr<3>(c.w[d], laneoff));
    }
  } else if constexpr (IB == 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint2 e;
      e = lds_u64(smem, perm_addr<0>(c.w[d], laneoff)); W[8 * d + 0] = e.x; W[8 * d + 1] = e.y;
      e = lds_u64(smem, perm_addr<1>(c.w[d], laneoff)); W[8 * d + 2] = e.x; W[8 * d + 3] = e.y;
      e = lds_u64(smem, perm_addr<2>(c.w[d], laneoff)); W[8 * d + 4] = e.x; W[8 * d + 5] = e.y;
      e = lds_u64(smem, perm_addr<3>(c.w[d], laneoff)); W[8 * d + 6] = e.x; W[8 * d + 7] = e.y;
    }
  } else if constexpr (IB == 1) {
    uint4 e;
    e = lds_u128(smem, perm_addr<0>(c.w[0], laneoff)); W[0] = e.x; W[1] = e.y; W[2] = e.z; W[3] = e.w;
    e = lds_u128(smem, perm_addr<1>(c.w[0], laneoff)); W[4] = e.x; W[5] = e.y; W[6] = e.z; W[7] = e.w;
    e = lds_u128(smem, perm_addr<2>(c.w[0], laneoff)); W[8] = e.x; W[9] = e.y; W[10] = e.z; W[11] = e.w;
    e = lds_u128(smem, perm_addr<3>(c.w[0], laneoff)); W[12] = e.x; W[13] = e.y; W[14] = e.z; W[15] = e.w;
  } else {  // IB == 3: 16 six-bit fields at bit 6p of the 96-bit chunk
    const uint32_t w0 = c.w[0], w1 = c.w[1], w2 = c.w[2];
    uint32_t f[16];
#pragma unroll
    for (int p = 0; p < 5; ++p) f[p] = (w0 >> (6 * p)) & 63u;
    f[5] = __builtin_amdgcn_alignbit(w1, w0, 30) & 63u;
#pragma unroll
    for (int p = 6; p < 10; ++p) f[p] = (w1 >> (6 * p - 32)) & 63u;
    f[10] = __builtin_amdgcn_alignbit(w2, w1, 28) & 63u;
#pragma unroll
    for (int p = 11; p < 16; ++p) f[p] = (w2 >> (6 * p - 64)) & 63u;
#pragma unroll
    for (int p = 0; p < 16; ++p) W[p] = lds_u32(smem, (f[p] << 8) | laneoff);
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

// IB: index bits (1..4).  BATCH: tokens per launch (1, 2, 4).  MAXCPL: most
// chunks a lane handles per row.  S: waves sharing one row (K split).
template <int IB, int BATCH, int MAXCPL, int S>
__global__ __launch_bounds__(kThreads) void cq_gemv_kernel(
    const uint8_t *__restrict__ idx, const uint16_t *__restrict__ norms,
    const int8_t *__restrict__ q, const float *__restrict__ scale, float *__restrict__ y,
    int rows, int cols, int plog2, int cpl, LevelTable T) {
  // Static LDS so the table base is a compile-time constant folded into the
  // ds_read offset field (a dynamic base costs one v_add per lookup).
  constexpr int TB = table_bytes<IB>();
  __shared__ __align__(16) uint8_t smem[TB];
  __shared__ float red[S > 1 ? kWavesPerBlock * kWave * BATCH : 1];   // [row slot][S][BATCH]

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int P = 1 << plog2;           // lanes per row slot
  const int rpw = kWave >> plog2;     // row slots per wave
  const int li = lane & (P - 1);
  const int rs = lane >> plog2;
  const int si = wave % S;            // which K part of the row this wave takes
  const int gw = wave / S;            // wave group within the block
  constexpr int groups_per_block = kWavesPerBlock / S;
  const int C = cols / kChunk;        // chunks per row
  const int ng = cols / kGroup;
  const int row_bytes = cols * IB / 8;
  const uint32_t laneoff = (uint32_t)(lane * entry_bytes<IB>()) & 255u;

  // ---- build the replicated lookup table
  for (int o = t * 16; o < TB; o += kThreads * 16) {
    *reinterpret_cast<uint4 *>(smem + o) = table_entry16<IB>(o >> 8, T);
  }

  // ---- this lane's activations as fp16 pairs, kept for every row
  uint32_t qh[BATCH][MAXCPL][16];
#pragma unroll
  for (int m = 0; m < MAXCPL; ++m) {
    const int c = li + P * (si * cpl + m);
    const bool ok = (m < cpl) && (c < C);
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      uint4 raw[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
      if (ok) {
        const uint4 *src = reinterpret_cast<const uint4 *>(q + (size_t)b * cols + c * kChunk);
        raw[0] = src[0];
        raw[1] = src[1];
      }
      const uint32_t wds[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w,
                               raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t word = wds[j >> 1];
        const int sh = (j & 1) * 16;
        const _Float16 lo = (_Float16)(int)(int8_t)(word >> sh);
        const _Float16 hi = (_Float16)(int)(int8_t)(word >> (sh + 8));
        h2 v = {lo, hi};
        qh[b][m][j] = __builtin_bit_cast(uint32_t, v);
      }
    }
  }
  __syncthreads();

  float post[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) post[b] = scale[b] * (T.cscale * (1.0f / kGroup));

  const int rows_per_iter = groups_per_block * rpw;
  for (int base = blockIdx.x * rows_per_iter; base < rows; base += gridDim.x * rows_per_iter) {
    const int row = base + gw * rpw + rs;
    const bool row_ok = row < rows;
    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;

    Chunk<IB> data[MAXCPL];
    float nrm[MAXCPL];
    const uint8_t *rp = idx + (size_t)row * row_bytes;
#pragma unroll
    for (int m = 0; m < MAXCPL; ++m) {
      const int c = li + P * (si * cpl + m);
      if (row_ok && m < cpl && c < C) {
        data[m] = load_chunk<IB>(rp + c * (4 * IB));
        nrm[m] = half_bits_to_float(norms[(size_t)row * ng + (c >> 2)]);
      }
    }
#pragma unroll
    for (int m = 0; m < MAXCPL; ++m) {
      const int c = li + P * (si * cpl + m);
      if (row_ok && m < cpl && c < C) {
        uint32_t W[16];
        lookup<IB>(data[m], smem, laneoff, W);
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; j += 2) {
            p0 = dot2(W[j], qh[b][m][j], p0);
            p1 = dot2(W[j + 1], qh[b][m][j + 1], p1);
          }
          acc[b] = fmaf(nrm[m], p0 + p1, acc[b]);
        }
      }
    }
    // reduce over the P lanes of the row slot
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      for (int off = P >> 1; off >= 1; off >>= 1) acc[b] += __shfl_xor(acc[b], off, 64);
    }
    if constexpr (S == 1) {
      if (row_ok && li == 0) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) y[(size_t)b * rows + row] = acc[b] * post[b];
      }
    } else {
      const int slot = gw * rpw + rs;
      if (li == 0) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) red[(slot * S + si) * BATCH + b] = acc[b];
      }
      __syncthreads();
      if (si == 0 && li == 0 && row_ok) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          float v = red[(slot * S) * BATCH + b];
          for (int k = 1; k < S; ++k) v += red[(slot * S + k) * BATCH + b];
          y[(size_t)b * rows + row] = v * post[b];
        }
      }
      __syncthreads();
    }
  }
}

struct GemvConfig {
  int plog2, cpl, S, maxcpl;
};

// Pick (lanes per row, chunks per lane, waves per row) so that every chunk of
// a row is covered and the lane's activation registers stay within budget.
bool choose_config(int C, int batch, GemvConfig &cfg) {
  const int budget = 8 / batch;   // chunks of fp16 pairs per lane: 16*budget*batch VGPRs
  for (int S = 1; S <= 8; S *= 2) {
    const int cw = (C + S - 1) / S;
    int P = 1, plog2 = 0;
    while (P < cw && P < kWave) { P <<= 1; ++plog2; }
    const int cpl = (cw + P - 1) / P;
    if (cpl <= budget) {
      cfg.plog2 = plog2;
      cfg.cpl = cpl;
      cfg.S = S;
      cfg.maxcpl = cpl <= 1 ? 1 : (cpl <= 2 ? 2 : (cpl <= 4 ? 4 : 8));
      return true;
    }
  }
  return false;
}

template <int IB, int BATCH, int MAXCPL, int S>
hipError_t launch_one(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      const int8_t *q, const float *scale, float *y, const GemvConfig &cfg,
                      int num_cus, hipStream_t s) {
  const int rpw = kWave >> cfg.plog2;
  const int rows_per_iter = (kWavesPerBlock / S) * rpw;
  int blocks = (L.rows + rows_per_iter - 1) / rows_per_iter;
  const int cap = 2 * num_cus;    // 64 KB of table per block: two blocks per CU
  if (blocks > cap) blocks = cap;
  const uint16_t *norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  cq_gemv_kernel<IB, BATCH, MAXCPL, S><<<blocks, kThreads, 0, s>>>(
      blob, norms, q, scale, y, L.rows, L.cols, cfg.plog2, cfg.cpl, T);
  return hipGetLastError();
}

template <int IB, int BATCH, int MAXCPL>
hipError_t dispatch_s(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      const int8_t *q, const float *scale, float *y, const GemvConfig &cfg,
                      int num_cus, hipStream_t s) {
  switch (cfg.S) {
    case 1: return launch_one<IB, BATCH, MAXCPL, 1>(blob, L, T, q, scale, y, cfg, num_cus, s);
    case 2: return launch_one<IB, BATCH, MAXCPL, 2>(blob, L, T, q, scale, y, cfg, num_cus, s);
    case 4: return launch_one<IB, BATCH, MAXCPL, 4>(blob, L, T, q, scale, y, cfg, num_cus, s);
    default: return launch_one<IB, BATCH, MAXCPL, 8>(blob, L, T, q, scale, y, cfg, num_cus, s);
  }
}

template <int IB, int BATCH>
hipError_t dispatch_cpl(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                        const int8_t *q, const float *scale, float *y, const GemvConfig &cfg,
                        int num_cus, hipStream_t s) {
  if constexpr (BATCH == 4) {
    if (cfg.maxcpl <= 1) return dispatch_s<IB, 4, 1>(blob, L, T, q, scale, y, cfg, num_cus, s);
    return dispatch_s<IB, 4, 2>(blob, L, T, q, scale, y, cfg, num_cus, s);
  } else if constexpr (BATCH == 2) {
    if (cfg.maxcpl <= 2) return dispatch_s<IB, 2, 2>(blob, L, T, q, scale, y, cfg, num_cus, s);
    return dispatch_s<IB, 2, 4>(blob, L, T, q, scale, y, cfg, num_cus, s);
  } else {
    if (cfg.maxcpl <= 2) return dispatch_s<IB, 1, 2>(blob, L, T, q, scale, y, cfg, num_cus, s);
    if (cfg.maxcpl <= 4) return dispatch_s<IB, 1, 4>(blob, L, T, q, scale, y, cfg, num_cus, s);
    return dispatch_s<IB, 1, 8>(blob, L, T, q, scale, y, cfg, num_cus, s);
  }
}

template <int IB>
hipError_t dispatch_batch(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int batch, float *y, int num_cus,
                          hipStream_t s) {
  // tokens in launches of up to four (weights are re-read per launch)
  const int C = L.cols / kChunk;
  for (int b0 = 0; b0 < batch;) {
    const int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    GemvConfig cfg;
    if (!choose_config(C, nb, cfg)) return hipErrorInvalidValue;
    const int8_t *qb = q + (size_t)b0 * L.cols;
    const float *sb = scale + b0;
    float *yb = y + (size_t)b0 * L.rows;
    hipError_t e;
    if (nb == 4) e = dispatch_cpl<IB, 4>(blob, L, T, qb, sb, yb, cfg, num_cus, s);
    else if (nb == 2) e = dispatch_cpl<IB, 2>(blob, L, T, qb, sb, yb, cfg, num_cus, s);
    else e = dispatch_cpl<IB, 1>(blob, L, T, qb, sb, yb, cfg, num_cus, s);
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

}  // namespace

bool cq_gemv_supported(int cols, int batch) {
  GemvConfig cfg;
  return choose_config(cols / kChunk, batch >= 4 ? 4 : (batch >= 2 ? 2 : 1), cfg);
}

hipError_t launch_cq_gemv(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int batch, float *y,
                          int num_cus, hipStream_t s) {
  switch (L.index_bits) {
    case 1: return dispatch_batch<1>(blob, L, T, q, scale, batch, y, num_cus, s);
    case 2: return dispatch_batch<2>(blob, L, T, q, scale, batch, y, num_cus, s);
    case 3: return dispatch_batch<3>(blob, L, T, q, scale, batch, y, num_cus, s);
    default: return dispatch_batch<4>(blob, L, T, q, scale, batch, y, num_cus, s);
  }
}

}  // namespace bqm
