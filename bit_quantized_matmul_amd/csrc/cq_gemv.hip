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

// Threads per workgroup: 1024 (128 VGPRs a wave) when a lane holds at most two
// chunks of a row, 512 (256 VGPRs) for longer rows so a wave can keep its
// current and next row of index words in registers.
template <int CPL> constexpr int block_threads() { return CPL >= 4 ? 512 : 1024; }
constexpr int kMaxWavesPerBlock = 16;
constexpr size_t kMaxActLds = 72 * 1024;   // LDS for the fp16 activations (table: 64 KB)
constexpr int kFusedScratch = 64 * 1024;   // fused: fp32 FWHT scratch, then the table
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

// Sum over all 64 lanes with DPP moves (no LDS round trips); the total
// lands in lanes 48..63.  Rotations inside each 16-lane row give every lane
// its row's sum; row_bcast15 / row_bcast31 then fold rows 0+1 and 2+3 into
// row 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}
// max of non-negative values over the wave (a 0 from a masked DPP row is harmless)
__device__ __forceinline__ float wave_max_to_lane63(float v) {
  v = fmaxf(v, dpp_f<0x121, 0xF>(v));
  v = fmaxf(v, dpp_f<0x122, 0xF>(v));
  v = fmaxf(v, dpp_f<0x124, 0xF>(v));
  v = fmaxf(v, dpp_f<0x128, 0xF>(v));
  v = fmaxf(v, dpp_f<0x142, 0xA>(v));
  v = fmaxf(v, dpp_f<0x143, 0xC>(v));
  return v;
}

__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f<0x121, 0xF>(v);   // row_ror:1
  v += dpp_f<0x122, 0xF>(v);   // row_ror:2
  v += dpp_f<0x124, 0xF>(v);   // row_ror:4
  v += dpp_f<0x128, 0xF>(v);   // row_ror:8
  v += dpp_f<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

struct GemvArgs {
  const uint8_t *idx;
  const uint16_t *norms;
  const int8_t *q;          // int8 activations [batch, cols]   (unfused)
  const float *scale;       // their per-token scales [batch]    (unfused)
  const float *x;           // fp32 activations [batch, cols]    (fused)
  int8_t *q_out;            // optional copy of the int8 codes   (fused)
  float *scale_out;         // optional copy of the scales       (fused)
  float *y;
  int rows, cols, plog2, nparts, rows_per_block;
};

// q = clip(rint(u / s), -127, 127) with u / s correctly rounded, computed as
// rint(u * inv) when that product is more than 1e-4 from a half-integer: for
// |u / s| <= 127 the product differs from the correctly rounded quotient by at
// most 2.3e-5, so both round to the same integer.  Otherwise the quotient is
// taken exactly.
__device__ __forceinline__ float a8_code(float u, float s, float inv) {
  const float yv = u * inv;
  float r = rintf(yv);
  if (fabsf(yv - floorf(yv) - 0.5f) < 1e-4f) r = rintf(__fdiv_rn(u, s));
  return fminf(fmaxf(r, -127.0f), 127.0f);
}

// Kernel shape: one persistent workgroup per CU, each taking a contiguous run
// of rows.  Setup per workgroup: the replicated lookup table and the
// activations as fp16 pairs in LDS (layout [batch][quarter][chunk][4 pairs],
// so lanes reading consecutive chunks hit consecutive 16-byte slots).  In the
// FUSED variant the workgroup first turns fp32 x into the int8 codes itself,
// with exactly the operations of act_fwht_quant_a8 (group FWHT in fp32, the
// row max, s = max / 127, the codes), while its first weight loads are in
// flight; the fp32 FWHT output is parked in the table's LDS before the table
// is built.
//
// A row slot of P lanes (P = 64, or fewer for short rows) owns a row.  The
// row's 32-index chunks are dealt out as slot s -> chunk li + P*s; a wave
// walks them as a sequence of work items, each one "part" of CPL slots of one
// row (NP parts per row), so registers stay bounded for any row length.  The
// accumulator carries across a row's parts; after the last part the row sum
// is reduced (DPP across the wave, or shuffles within a short row slot) and
// stored.  S > 1 splits a row across S waves (used only when there are too
// few rows to occupy the GPU; then NP == 1) and meets in LDS.
//
// Loads are issued unconditionally and one work item ahead: each chunk's
// registers are refilled with the next item's chunk right after use.  Past
// the end they read valid bytes (the block's last row, chunk 0) and are
// weighted by a zero norm.  With QREG the lane keeps its fp16 activation
// pairs in registers (filled once from LDS), otherwise it re-reads them from
// LDS per chunk.
//
// IB: index bits (1..4).  BATCH: tokens per launch (1, 2, 4).  CPL: chunks a
// lane handles per work item.  QREG: activations in registers (NP == 1).
// S: waves per row.  FULL: P == 64 (the row sum reduces with DPP).
// FUSED: fp32 activations in, A8 done in the prologue.
template <int IB, int BATCH, int CPL, bool QREG, int S, bool FULL, bool FUSED>
__global__ __launch_bounds__(block_threads<CPL>()) void cq_gemv_kernel(GemvArgs A, LevelTable T) {
  constexpr int TB = table_bytes<IB>();
  constexpr int TAB_BYTES = FUSED ? kFusedScratch : TB;   // fused: also the FWHT scratch
  constexpr int kThreads = block_threads<CPL>();
  constexpr int kWavesPerBlock = kThreads / kWave;
  __shared__ __align__(16) uint8_t tab[TAB_BYTES];
  __shared__ float red[S > 1 ? kThreads / kWave * kWave * BATCH : 1];
  __shared__ float amax_red[FUSED ? kWavesPerBlock * BATCH : 1];
  __shared__ float s_fused[BATCH];
  extern __shared__ __align__(16) uint32_t qs[];        // fp16 pairs, see layout above

  const int rows = A.rows, cols = A.cols;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int P = FULL ? kWave : (1 << A.plog2);
  const int rpw = FULL ? 1 : (kWave >> A.plog2);
  const int li = FULL ? lane : (lane & (P - 1));
  const int rs = FULL ? 0 : (lane >> A.plog2);
  const int si = wave % S;
  const int gw = wave / S;
  const int nparts = A.nparts;
  constexpr int groups = kWavesPerBlock / S;
  const int C = cols / kChunk;
  const int ng = cols / kGroup;
  const int row_bytes = cols * IB / 8;
  const uint32_t laneoff = (uint32_t)(lane * entry_bytes<IB>()) & 255u;
  const int r0 = blockIdx.x * A.rows_per_block;
  const int r1 = min(rows, r0 + A.rows_per_block);
  const int rows_per_iter = groups * rpw;
  const uint8_t *idx = A.idx;
  const uint32_t *norm_words = reinterpret_cast<const uint32_t *>(A.norms);

  // chunk of slot m in part `part` (this lane), and whether it exists
  auto chunk_of = [&](int part, int m) { return li + P * ((si * nparts + part) * CPL + m); };
  auto clamp_row = [&](int row) { return row < r1 ? row : r1 - 1; };
  // Index words and the 32-bit word holding the chunk's fp16 norm (a 16-bit
  // load would be packed with its neighbour, and packing waits for the load).
  auto load_one = [&](int row, int part, int m, Chunk<IB> &d, uint32_t &nword) {
    const int rr = clamp_row(row);
    const int c0 = chunk_of(part, m);
    const int cc = c0 < C ? c0 : 0;
    d = load_chunk<IB>(idx + (size_t)rr * row_bytes + cc * (4 * IB));
    nword = norm_words[((size_t)rr * ng + (cc >> 2)) >> 1];
  };

  // the first work item's loads go out before the setup work
  int row = r0 + gw * rpw + rs;
  int part = 0;
  Chunk<IB> cur[CPL];
  uint32_t ncur[CPL];
#pragma unroll
  for (int m = 0; m < CPL; ++m) load_one(row, 0, m, cur[m], ncur[m]);

  auto store_pair = [&](int b, int p_lin, uint32_t pr) {   // p_lin: pair index within the row
    const int c = p_lin >> 4, p = p_lin & 15;
    qs[((b * 4 + (p >> 2)) * C + c) * 4 + (p & 3)] = pr;
  };

  if constexpr (FUSED) {
    // ---- A8 on fp32 x: FWHT per 128-group (8 elements a lane, 16 lanes a
    // group), the same network and fp32 operations as act_fwht_quant_a8
    float *ubuf = reinterpret_cast<float *>(tab);
    const int c8 = cols / 8;
    float lmax[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      lmax[b] = 0.0f;
      for (int ci = t; ci < c8; ci += kThreads) {
        const float *xp = A.x + (size_t)b * cols + 8 * ci;
        const float4 xa = *reinterpret_cast<const float4 *>(xp);
        const float4 xb = *reinterpret_cast<const float4 *>(xp + 4);
        float v[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if ((j & h) == 0) {
              const float a = v[j], c = v[j + h];
              v[j] = a + c;
              v[j + h] = a - c;
            }
          }
        }
#pragma unroll
        for (int hl = 1; hl < 16; hl <<= 1) {
          const bool upper = (lane & hl) != 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float other = __shfl_xor(v[e], hl, 64);
            v[e] = upper ? (other - v[e]) : (v[e] + other);
          }
        }
        float4 *up = reinterpret_cast<float4 *>(ubuf + b * cols + 8 * ci);
        up[0] = make_float4(v[0], v[1], v[2], v[3]);
        up[1] = make_float4(v[4], v[5], v[6], v[7]);
#pragma unroll
        for (int e = 0; e < 8; ++e) lmax[b] = fmaxf(lmax[b], fabsf(v[e]));
      }
      lmax[b] = wave_max_to_lane63(lmax[b]);
      if (lane == 63) amax_red[b * kWavesPerBlock + wave] = lmax[b];
    }
    __syncthreads();
    if (t < BATCH) {
      float mx = amax_red[t * kWavesPerBlock];
      for (int w = 1; w < kWavesPerBlock; ++w) mx = fmaxf(mx, amax_red[t * kWavesPerBlock + w]);
      const float sc = (mx > 0.0f) ? __fdiv_rn(mx, 127.0f) : 1.0f;
      s_fused[t] = sc;
      if (blockIdx.x == 0 && A.scale_out) A.scale_out[t] = sc;
    }
    __syncthreads();
    const int quads = cols / 4;
    for (int e = t; e < BATCH * quads; e += kThreads) {
      const int b = e / quads, w = e - b * quads;
      const float sc = s_fused[b];
      const float inv = 1.0f / sc;
      const float4 u = reinterpret_cast<const float4 *>(ubuf + b * cols)[w];
      const float c0 = a8_code(u.x, sc, inv), c1 = a8_code(u.y, sc, inv);
      const float c2 = a8_code(u.z, sc, inv), c3 = a8_code(u.w, sc, inv);
      h2 p0 = {(_Float16)c0, (_Float16)c1};
      h2 p1 = {(_Float16)c2, (_Float16)c3};
      store_pair(b, 2 * w, __builtin_bit_cast(uint32_t, p0));
      store_pair(b, 2 * w + 1, __builtin_bit_cast(uint32_t, p1));
      if (blockIdx.x == 0 && A.q_out) {
        const uint32_t packed = ((uint32_t)(uint8_t)(int8_t)(int)c0) |
                                ((uint32_t)(uint8_t)(int8_t)(int)c1 << 8) |
                                ((uint32_t)(uint8_t)(int8_t)(int)c2 << 16) |
                                ((uint32_t)(uint8_t)(int8_t)(int)c3 << 24);
        reinterpret_cast<uint32_t *>(A.q_out + (size_t)b * cols)[w] = packed;
      }
    }
    __syncthreads();                       // ubuf is dead: the table may overwrite it
  } else {
    // int8 -> fp16 pairs: dword w of row b holds q[b][4w .. 4w+3] = pairs 2w, 2w+1
    const int words = cols / 4;
    for (int e = t; e < BATCH * words; e += kThreads) {
      const int b = e / words, w = e - b * words;
      const uint32_t v = reinterpret_cast<const uint32_t *>(A.q + (size_t)b * cols)[w];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const _Float16 lo = (_Float16)(int)(int8_t)(v >> (16 * h));
        const _Float16 hi = (_Float16)(int)(int8_t)(v >> (16 * h + 8));
        h2 pr = {lo, hi};
        store_pair(b, 2 * w + h, __builtin_bit_cast(uint32_t, pr));
      }
    }
  }
  for (int o = t * 16; o < TB; o += kThreads * 16)
    *reinterpret_cast<uint4 *>(tab + o) = table_entry16<IB>(o >> 8, T);
  __syncthreads();

  auto qpairs = [&](int b, int c, uint32_t (&out)[16]) {      // c: chunk index (< C)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4 *>(&qs[((b * 4 + i) * C + c) * 4]);
      out[4 * i + 0] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  };
  uint32_t qreg[QREG ? BATCH : 1][QREG ? CPL : 1][16];
  if constexpr (QREG) {
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        const int c = chunk_of(0, m);
        qpairs(b, c < C ? c : 0, qreg[b][m]);
      }
  }

  float post[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b)
    post[b] = (FUSED ? s_fused[b] : A.scale[b]) * (T.cscale * (1.0f / kGroup));

  float acc[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
  const int items = ((r1 - r0 + rows_per_iter - 1) / rows_per_iter) * nparts;
  for (int it = 0; it < items; ++it) {
    const bool last_part = part == nparts - 1;
    const int nrow = last_part ? row + rows_per_iter : row;
    const int npart = last_part ? 0 : part + 1;
    const bool live = row < r1;
    const int rbase = clamp_row(row) * ng;
    // software pipeline over the item's chunks: the lookups of chunk m+1 are
    // in flight while chunk m's dot products run; sched_barrier keeps the
    // compiler from hoisting further (which would blow the register budget)
    uint32_t Wn[16];
    lookup<IB>(cur[0], tab, laneoff, Wn);
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      uint32_t W[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) W[j] = Wn[j];
      if (m + 1 < CPL) lookup<IB>(cur[m + 1], tab, laneoff, Wn);
      const int c0 = chunk_of(part, m);
      const bool cok = c0 < C;
      const int cc = cok ? c0 : 0;
      const uint32_t sh = (uint32_t)((rbase + (cc >> 2)) & 1) * 16u;
      const float nv = (live && cok) ? half_bits_to_float((uint16_t)(ncur[m] >> sh)) : 0.0f;
      load_one(nrow, npart, m, cur[m], ncur[m]);       // refill with the next item's chunk
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        uint32_t qq[16];
        if constexpr (QREG) {
#pragma unroll
          for (int j = 0; j < 16; ++j) qq[j] = qreg[b][m][j];
        } else {
          qpairs(b, cc, qq);
        }
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          p0 = dot2(W[j], qq[j], p0);
          p1 = dot2(W[j + 1], qq[j + 1], p1);
        }
        acc[b] = fmaf(nv, p0 + p1, acc[b]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last_part) {                     // uniform across the workgroup
      bool writer;
      if constexpr (FULL) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[b] = wave_sum_to_lane63(acc[b]);
        writer = lane == 63;
      } else {
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
          for (int off = P >> 1; off >= 1; off >>= 1) acc[b] += __shfl_xor(acc[b], off, 64);
        writer = li == 0;
      }
      if constexpr (S == 1) {
        if (live && writer) {
#pragma unroll
          for (int b = 0; b < BATCH; ++b) A.y[(size_t)b * rows + row] = acc[b] * post[b];
        }
      } else {
        const int slot = gw * rpw + rs;
        if (writer) {
#pragma unroll
          for (int b = 0; b < BATCH; ++b) red[(slot * S + si) * BATCH + b] = acc[b];
        }
        __syncthreads();
        if (si == 0 && writer && live) {
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            float v = red[(slot * S) * BATCH + b];
            for (int k = 1; k < S; ++k) v += red[(slot * S + k) * BATCH + b];
            A.y[(size_t)b * rows + row] = v * post[b];
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
    }
    row = nrow;
    part = npart;
  }
}

struct GemvConfig {
  int plog2, cpl, S, nparts;
  bool qreg;
};

// Lanes per row slot P (a power of two up to 64), chunks per lane per work
// item CPL (1, 2 or 4), parts per row NP and waves per row S, so that
// P * CPL * NP * S covers the row's C chunks.  The K split S is used only
// when rows are too few to give the GPU's waves work; it needs NP == 1.
bool choose_config(int rows, int C, int batch, int num_cus, GemvConfig &cfg) {
  const int waves_total = num_cus * 8;
  const int max_cpl = batch >= 4 ? 2 : 4;
  for (int S = 1; S <= 8; S *= 2) {
    const int cw = (C + S - 1) / S;
    int P = 1, plog2 = 0;
    while (P < cw && P < kWave) { P <<= 1; ++plog2; }
    const int slots = (cw + P - 1) / P;                 // chunks a lane owns in a row
    const int rpw = kWave / P;
    const long wave_rows = ((long)rows * S + rpw - 1) / rpw;
    if (S < 8 && wave_rows < waves_total) continue;      // too little parallelism: split K
    int cpl = slots <= 1 ? 1 : (slots <= 2 ? 2 : 4);
    if (cpl > max_cpl) cpl = max_cpl;
    const int nparts = (slots + cpl - 1) / cpl;
    if (S > 1 && nparts > 1) continue;
    cfg.plog2 = plog2;
    cfg.cpl = cpl;
    cfg.S = S;
    cfg.nparts = nparts;
    cfg.qreg = nparts == 1 && cpl * batch <= 2;
    return true;
  }
  // long rows and few of them: no K split, parts instead
  const int cw = C;
  const int P = kWave;
  const int slots = (cw + P - 1) / P;
  int cpl = slots <= 1 ? 1 : (slots <= 2 ? 2 : 4);
  if (cpl > max_cpl) cpl = max_cpl;
  cfg.plog2 = 6;
  cfg.cpl = cpl;
  cfg.S = 1;
  cfg.nparts = (slots + cpl - 1) / cpl;
  cfg.qreg = false;
  return true;
}

template <int IB, int BATCH, int CPL, bool QREG, int S, bool FUSED>
hipError_t launch_one(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      GemvArgs A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  constexpr int kThreads = block_threads<CPL>();
  constexpr int kWavesPerBlock = kThreads / kWave;
  const int rpw = kWave >> cfg.plog2;
  const int rows_per_iter = (kWavesPerBlock / S) * rpw;
  int blocks = (L.rows + rows_per_iter - 1) / rows_per_iter;
  if (blocks > num_cus) blocks = num_cus;
  const int rpb = (L.rows + blocks - 1) / blocks;   // rows per block (the tail iteration is partial)
  blocks = (L.rows + rpb - 1) / rpb;
  const size_t qbytes = (size_t)BATCH * L.cols * 2;
  A.idx = blob;
  A.norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  A.rows = L.rows;
  A.cols = L.cols;
  A.plog2 = cfg.plog2;
  A.nparts = cfg.nparts;
  A.rows_per_block = rpb;
  if constexpr (CPL == 1) {
    // rows shorter than 64 chunks: several rows per wave (only ever one chunk per lane)
    if (cfg.plog2 < 6) {
      cq_gemv_kernel<IB, BATCH, CPL, QREG, S, false, FUSED><<<blocks, kThreads, qbytes, s>>>(A, T);
      return hipGetLastError();
    }
  }
  cq_gemv_kernel<IB, BATCH, CPL, QREG, S, true, FUSED><<<blocks, kThreads, qbytes, s>>>(A, T);
  return hipGetLastError();
}

template <int IB, int BATCH, int CPL, bool QREG, bool FUSED>
hipError_t dispatch_s(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      const GemvArgs &A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  switch (cfg.S) {
    case 1: return launch_one<IB, BATCH, CPL, QREG, 1, FUSED>(blob, L, T, A, cfg, num_cus, s);
    case 2: return launch_one<IB, BATCH, CPL, QREG, 2, FUSED>(blob, L, T, A, cfg, num_cus, s);
    case 4: return launch_one<IB, BATCH, CPL, QREG, 4, FUSED>(blob, L, T, A, cfg, num_cus, s);
    default: return launch_one<IB, BATCH, CPL, QREG, 8, FUSED>(blob, L, T, A, cfg, num_cus, s);
  }
}

template <int IB, int BATCH, int CPL, bool FUSED>
hipError_t dispatch_q(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      const GemvArgs &A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  if constexpr (CPL * BATCH <= 2) {
    if (cfg.qreg) return dispatch_s<IB, BATCH, CPL, true, FUSED>(blob, L, T, A, cfg, num_cus, s);
  }
  return dispatch_s<IB, BATCH, CPL, false, FUSED>(blob, L, T, A, cfg, num_cus, s);
}

template <int IB, int BATCH, bool FUSED>
hipError_t dispatch_cpl(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                        const GemvArgs &A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  if (cfg.cpl == 1) return dispatch_q<IB, BATCH, 1, FUSED>(blob, L, T, A, cfg, num_cus, s);
  if constexpr (BATCH >= 4) {
    return dispatch_q<IB, BATCH, 2, FUSED>(blob, L, T, A, cfg, num_cus, s);
  } else {
    if (cfg.cpl == 2) return dispatch_q<IB, BATCH, 2, FUSED>(blob, L, T, A, cfg, num_cus, s);
    return dispatch_q<IB, BATCH, 4, FUSED>(blob, L, T, A, cfg, num_cus, s);
  }
}

// Tokens go in launches of up to four (weights are re-read per launch).  The
// fp16 copy of a launch's activations must fit in LDS beside the table; in
// the fused variant their fp32 FWHT must also fit the table's 64 KB.
template <int IB, bool FUSED>
hipError_t dispatch_batch(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, const float *x, int8_t *q_out,
                          float *scale_out, int batch, float *y, int num_cus, hipStream_t s) {
  const int C = L.cols / kChunk;
  for (int b0 = 0; b0 < batch;) {
    int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    while (nb > 1 && ((size_t)nb * L.cols * 2 > kMaxActLds ||
                      (FUSED && (size_t)nb * L.cols * 4 > (size_t)kFusedScratch)))
      nb >>= 1;
    GemvConfig cfg;
    if (!choose_config(L.rows, C, nb, num_cus, cfg)) return hipErrorInvalidValue;
    GemvArgs A{};
    A.q = q ? q + (size_t)b0 * L.cols : nullptr;
    A.scale = scale ? scale + b0 : nullptr;
    A.x = x ? x + (size_t)b0 * L.cols : nullptr;
    A.q_out = q_out ? q_out + (size_t)b0 * L.cols : nullptr;
    A.scale_out = scale_out ? scale_out + b0 : nullptr;
    A.y = y + (size_t)b0 * L.rows;
    hipError_t e;
    if (nb == 4) e = dispatch_cpl<IB, 4, FUSED>(blob, L, T, A, cfg, num_cus, s);
    else if (nb == 2) e = dispatch_cpl<IB, 2, FUSED>(blob, L, T, A, cfg, num_cus, s);
    else e = dispatch_cpl<IB, 1, FUSED>(blob, L, T, A, cfg, num_cus, s);
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

}  // namespace

bool cq_gemv_supported(int cols, int batch, bool fused) {
  (void)batch;
  GemvConfig cfg;
  if (cols % kChunk) return false;
  if ((size_t)cols * 2 > kMaxActLds) return false;       // one token's fp16 copy must fit
  if (fused && (size_t)cols * 4 > (size_t)kFusedScratch) return false;
  return choose_config(1 << 20, cols / kChunk, 1, 256, cfg);
}

hipError_t launch_cq_gemv(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int batch, float *y,
                          int num_cus, hipStream_t s) {
  switch (L.index_bits) {
    case 1: return dispatch_batch<1, false>(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
    case 2: return dispatch_batch<2, false>(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
    case 3: return dispatch_batch<3, false>(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
    default: return dispatch_batch<4, false>(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
  }
}

hipError_t launch_cq_gemv_f32(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                              const float *x, int batch, float *y, int8_t *q_out,
                              float *scale_out, int num_cus, hipStream_t s) {
  switch (L.index_bits) {
    case 1: return dispatch_batch<1, true>(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
    case 2: return dispatch_batch<2, true>(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
    case 3: return dispatch_batch<3, true>(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
    default: return dispatch_batch<4, true>(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
  }
}

}  // namespace bqm
