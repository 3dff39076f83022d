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
#pragma once
#include "bqm_common.h"

namespace bqm {
namespace {

// Threads per workgroup: 1024 (128 VGPRs a wave) when a lane holds at most two
// chunks of a row, 512 (256 VGPRs) for longer rows so a wave can keep its
// current and next row of index words in registers.
template <int CPL> constexpr int block_threads() { return CPL >= 4 ? 512 : 1024; }
constexpr size_t kMaxActLds = 72 * 1024;   // LDS for the fp16 activations (table: 64 KB)
constexpr int kMaxFusedCols = 16384;       // fused A8: the widest row (registers hold its 16-element segments)
constexpr int kRingChunks = 8;             // 32-index chunks a lane keeps in flight
constexpr int kMaxRowsBlk = 512;           // rows x K-split waves a workgroup finishes
constexpr uint32_t kOOB = 0x80000000u;     // buffer offset past every range: reads give 0
constexpr uint32_t kIdxLimit = 1u << 30;   // packed bytes addressable through one descriptor
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer descriptor word 3 on gfx9
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int IB>
struct Chunk;   // raw index bytes of one 32-index chunk
template <> struct Chunk<1> { uint32_t w[1]; };
template <> struct Chunk<2> { uint32_t w[2]; };
template <> struct Chunk<3> { uint32_t w[3]; };
template <> struct Chunk<4> { uint32_t w[4]; };

// Raw buffer descriptor over [base, base + bytes).  Loads at offsets past the
// range return zeros without touching memory, which is how the kernels read
// past the end of a matrix or a block's rows: the offset is replaced by kOOB.
// (Only the per-lane offset and the instruction offset are range-checked, so
// the whole offset is always passed per lane.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
constexpr int kNT = 2;   // cache policy: non-temporal (weights are read once)

template <int IB>
__device__ __forceinline__ Chunk<IB> load_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Chunk<IB> c;
  if constexpr (IB == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else if constexpr (IB == 3) {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, kNT));
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z;
  } else if constexpr (IB == 2) {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT));
    c.w[0] = v.x; c.w[1] = v.y;
  } else {
    c.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNT);
  }
  return c;
}

// The aligned 32-bit word holding the fp16 norm at byte offset `off` (the half
// is picked at use).  A 16-bit load would be widened or packed with its
// neighbour right after the load, which makes the compiler wait for it there.
__device__ __forceinline__ uint32_t load_norm_word(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off & ~3u, 0, 0);
}

// Table bytes and entry size per index width.
template <int IB> constexpr int table_rows() { return IB == 3 ? 64 : 256; }
template <int IB> constexpr int entry_bytes() { return IB == 1 ? 16 : (IB == 2 ? 8 : 4); }
template <int IB> constexpr int table_bytes() { return table_rows<IB>() * 256; }

// Levels (fp16 bits) of table row `e`, packed as the row's entry (16 bytes:
// the entry replicated).  `lv(i)` gives the fp16 bits of level i.
template <int IB, class LV>
__device__ __forceinline__ uint4 table_entry16(int e, LV lv) {
  if constexpr (IB == 4 || IB == 3) {
    const int lo = (IB == 4) ? (e & 15) : (e & 7);
    const int hi = (IB == 4) ? (e >> 4) : (e >> 3);
    const uint32_t v = lv(lo) | (lv(hi) << 16);
    return make_uint4(v, v, v, v);
  } else if constexpr (IB == 2) {
    const uint32_t a = lv(e & 3) | (lv((e >> 2) & 3) << 16);
    const uint32_t b = lv((e >> 4) & 3) | (lv((e >> 6) & 3) << 16);
    return make_uint4(a, b, a, b);
  } else {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = lv((e >> (2 * j)) & 1) | (lv((e >> (2 * j + 1)) & 1) << 16);
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
  int rows, cols, plog2, nparts, S, rows_per_block;
  uint32_t idx_bytes, norm_bytes, act_bytes;
};

// q = clip(rint(u / s), -127, 127) with u / s correctly rounded, computed as
// rint(u * inv), inv = rcp(s) (within 1 ulp of 1 / s), unless u * inv lies
// within 1e-4 of a half-integer: for |u / s| <= 127 the product differs from
// the correctly rounded quotient by at most 2.3e-5, so away from the rounding
// boundaries both give the same integer.  Near a boundary (rare) the quotient
// is taken exactly.  The distance test is one maximum over the lanes'
// elements.  The clip binds only when s is subnormal (for a normal
// s = RN(amax / 127), |u| / s <= 127 (1 + 2^-23) rounds to at most 127), so it
// runs only then (`clip`, uniform).
template <int N>
__device__ __forceinline__ void a8_codes(const float (&u)[N], float s, float inv, bool clip,
                                         float (&code)[N]) {
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    code[i] = rintf(u[i] * inv);
    dmax = fmaxf(dmax, fabsf(fmaf(u[i], inv, -code[i])));
  }
  if (dmax > 0.4999f) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (fabsf(fmaf(u[i], inv, -code[i])) > 0.4999f) code[i] = rintf(__fdiv_rn(u[i], s));
    }
  }
  if (clip) {
#pragma unroll
    for (int i = 0; i < N; ++i) code[i] = __builtin_amdgcn_fmed3f(code[i], -127.0f, 127.0f);
  }
}

// DPP quad permutations: lane i reads lane i^1 / i^2 of its group of four.
__device__ __forceinline__ float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
}
// Lane i reads lane i^4 of its group of eight: the half-row mirror (i -> 7 - i)
// followed by the quad reversal (i -> i ^ 3).
__device__ __forceinline__ float oct_xor4(float v) {
  const int m = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true);
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true));
}
// Lane i reads lane i^8 of its row of sixteen: the row rotated by 8.
__device__ __forceinline__ float row_xor8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
}

// Kernel shape: at most one workgroup per CU (more only for very tall
// matrices), each finishing a contiguous run of rows.
//
// The hardware retires vector loads in order, and the compiler waits for one
// particular load precisely only if every load is issued on every path: a
// load under a branch makes it wait for all of them.  The kernel is laid out
// around that:
//  1. each wave issues its first work item's loads, then (only waves that own
//     activations) the activation loads, builds its rows of the replicated
//     lookup table, and waits for everything issued so far (one round trip,
//     overlapped with the table);
//  2. the next PD - 1 work items' loads go out, unconditionally;
//  3. activations -> fp16 pairs in LDS (layout [batch][quarter][chunk][4
//     pairs], so lanes reading consecutive chunks hit consecutive 16-byte
//     slots); block barrier;
//  4. main loop: process item i (waiting for exactly its loads), then refill
//     its ring slot with item i + PD.  Items past a wave's end read at offset
//     kOOB (zeros, no memory traffic).  Row sums go to LDS, never to global
//     memory inside the loop (stores share the load counter);
//  5. after a barrier the block adds the S K-split partials of each row in a
//     fixed order and writes y with coalesced stores.
//
// FUSED runs the A8 step on fp32 x with the same fp32 operations as
// act_fwht_quant_a8: a thread holds KSEG-element segments of a group in
// registers (16, or 8 for one token past 8192 columns), runs the in-register
// butterfly stages (4, or 3), then the stages across the lanes of the group
// (8 lanes: 3 stages, or 16 lanes: 4) with DPP permutations (every butterfly
// is the same a + b, a - b on the same operands, so the values match the
// other kernel's bit for bit); block max, s = max / 127, and the codes go
// straight from registers to LDS.
//
// Work split: a row slot of P lanes (P = 64, or fewer for short rows) owns a
// row; its 32-index chunks are dealt out as slot s -> chunk li + P * s.  A
// wave walks a sequence of work items, each one "part" of CPL slots of one
// row (NP parts per row); with a K split the S waves of a group share rows.
//
// IB: index bits (1..4).  BATCH: tokens per launch (1, 2, 4).  CPL: chunks a
// lane handles per work item.  QREG: activations held in registers (NP == 1).
// PD: work items in flight per wave.  FULL: P == 64 (the row sum reduces with
// DPP).  FUSED: fp32 activations in, A8 done in the prologue.  KSEG: the
// fused prologue's segment length (16 or 8).
template <int IB, int BATCH, int CPL, bool QREG, int PD, bool FULL, bool FUSED, int KSEG>
__global__ __launch_bounds__(block_threads<CPL>()) void cq_gemv_kernel(GemvArgs A, LevelTable T) {
  constexpr int TB = table_bytes<IB>();
  constexpr int kThreads = block_threads<CPL>();
  constexpr int kWaves = kThreads / kWave;
  constexpr int kCB = 4 * IB;                       // bytes of one chunk
  static_assert(FULL || CPL == 1, "short row slots take one chunk per item");
  constexpr int kSeg = KSEG;                        // fused A8: elements a thread holds per segment
  constexpr int SEGS = FUSED ? (BATCH * kMaxFusedCols / kSeg + kThreads - 1) / kThreads : 1;
  constexpr int QV = FUSED ? 1 : (int)((kMaxActLds / 2 + 16 * kThreads - 1) / (16 * kThreads));
  __shared__ __align__(16) uint8_t tab[TB];
  __shared__ float yblk[kMaxRowsBlk * BATCH];
  __shared__ float amax_red[FUSED ? kWaves * BATCH : 1];
  __shared__ float s_blk[2 * BATCH];                // scale, 1 / scale
  extern __shared__ __align__(16) uint32_t qs[];    // fp16 pairs, see layout above

  const int rows = A.rows, cols = A.cols;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: the row math is scalar
  const int S = A.S;                                // waves per row (divides kWaves)
  const int P = FULL ? kWave : (1 << A.plog2);
  const int rpw = FULL ? 1 : (kWave >> A.plog2);
  const int li = FULL ? lane : (lane & (P - 1));
  const int rs = FULL ? 0 : (lane >> A.plog2);
  const int si = wave % S;
  const int gw = wave / S;
  const int nparts = A.nparts;
  const int groups = kWaves / S;
  const int C = cols / kChunk;
  const int ng = cols / kGroup;
  const int row_bytes = cols * IB / 8;
  const uint32_t laneoff = (uint32_t)(lane * entry_bytes<IB>()) & 255u;
  const int r0 = blockIdx.x * A.rows_per_block;
  const int r1 = min(rows, r0 + A.rows_per_block);
  const int rows_per_iter = groups * rpw;
  const int iters = (r1 - r0 + rows_per_iter - 1) / rows_per_iter;
  const int NI = iters * nparts;                    // work items of every wave in the block

  const __amdgpu_buffer_rsrc_t ridx = make_rsrc(A.idx, A.idx_bytes);
  const __amdgpu_buffer_rsrc_t rnrm = make_rsrc(A.norms, A.norm_bytes);
  const __amdgpu_buffer_rsrc_t ract =
      make_rsrc(FUSED ? (const void *)A.x : (const void *)A.q, A.act_bytes);

  // lanes 0..15 hold the fp16 bits of levels 0..15 (selected from the scalar
  // kernel arguments, so building the table waits on no vector load)
  int lv_lane = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) lv_lane = (lane == i) ? (int)T.h16[i] : lv_lane;

  // work item (k, part) -> ring slot; items past the wave's end read zeros.
  // FULL: the wave's row of an item is read through descriptors whose range
  // is that row (empty for items past the wave's end), so chunks past the
  // row's end read zeros without traffic and the per-lane offsets are fixed;
  // the norm descriptor covers the aligned words holding the row's norms
  // (never past the norm region: its end is 64-byte aligned).
  const uint32_t lane_idx = (uint32_t)(rs * row_bytes + li * kCB);
  const uint32_t lane_nrm = (uint32_t)(li >> 2) * 2u;                 // FULL: rs == 0
  auto issue = [&](int k, int part, Chunk<IB> (&dst)[CPL], uint32_t (&ndst)[CPL]) {
    const int rbase = r0 + gw * rpw + k * rows_per_iter;         // row of this lane: rbase + rs
    const bool live = (k < iters) && (rbase + rs < r1);
    const int sbase = (si * nparts + part) * CPL;                // first slot of the item
    if constexpr (FULL) {
      const uint32_t nrow = (uint32_t)rbase * (uint32_t)ng;       // the row's first norm
      const uint32_t adj = (nrow & 1u) * 2u;                      // its byte offset in its word
      const __amdgpu_buffer_rsrc_t ri =
          make_rsrc(A.idx + (size_t)rbase * row_bytes, live ? (uint32_t)row_bytes : 0u);
      const __amdgpu_buffer_rsrc_t rn =
          make_rsrc(A.norms + (nrow & ~1u), live ? ((uint32_t)(2 * ng) + adj + 3u) & ~3u : 0u);
      const uint32_t oi = lane_idx + (uint32_t)(sbase * P * kCB);
      const uint32_t on = lane_nrm + adj + (uint32_t)(sbase * (P / 2));
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        dst[m] = load_chunk<IB>(ri, oi + (uint32_t)(m * P * kCB));
        ndst[m] = load_norm_word(rn, on + (uint32_t)(m * (P / 2)));
      }
      return;
    }
    uint32_t vi = (uint32_t)rbase * (uint32_t)row_bytes + lane_idx + (uint32_t)(sbase * P * kCB);
    // norm of chunk c = li + P * slot is that of group c / 4; with P = 64 the
    // group of slot m is the group of slot 0 plus 16 m (short row slots have
    // CPL == 1 and P possibly < 4, so the group is formed exactly)
    uint32_t vn;
    if constexpr (FULL)
      vn = (uint32_t)rbase * (uint32_t)ng * 2u + lane_nrm + (uint32_t)(sbase * (P / 2));
    else
      vn = ((uint32_t)(rbase + rs) * (uint32_t)ng + (uint32_t)((li + P * sbase) >> 2)) * 2u;
    vi = live ? vi : kOOB;
    vn = live ? vn : kOOB;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      dst[m] = load_chunk<IB>(ridx, vi + (uint32_t)(m * P * kCB));
      ndst[m] = load_norm_word(rnrm, vn + (uint32_t)(m * (P / 2)));
    }
  };
  auto advance = [&](int &k, int &part) {
    if (++part == nparts) { part = 0; ++k; }
  };
  Chunk<IB> ring[PD][CPL];
  uint32_t nring[PD][CPL];
  int ik = 0, ipart = 0;

  // ---- 1. activations, then the first work item, table, one wait (for the
  // activations only: the first item's 2 CPL loads may still be in flight)
  float xv[SEGS][FUSED ? kSeg : 1];
  u32x4 qv[QV];
  uint32_t sclw[BATCH];
  const int nseg = BATCH * (cols / kSeg);           // 16-element segments (fused)
  const int nq = BATCH * cols;                      // int8 codes (unfused)
  if constexpr (FUSED) {
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      if (wave * kWave + j * kThreads >= nseg) continue;   // wave-uniform
      const uint32_t base = (uint32_t)(t + j * kThreads) * (4u * kSeg);
#pragma unroll
      for (int e = 0; e < kSeg / 4; ++e) {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ract, base + 16 * e, 0, 0));
        xv[j][4 * e + 0] = __uint_as_float(w.x);
        xv[j][4 * e + 1] = __uint_as_float(w.y);
        xv[j][4 * e + 2] = __uint_as_float(w.z);
        xv[j][4 * e + 3] = __uint_as_float(w.w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < QV; ++j) {
      if ((wave * kWave + j * kThreads) * 16 >= nq) continue;   // wave-uniform
      qv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            ract, (uint32_t)(t + j * kThreads) * 16u, 0, 0));
    }
    // the scales: a vector load (every lane the same address); a scalar load
    // would be waited for by every later LDS wait (they share one counter)
    const __amdgpu_buffer_rsrc_t rscl = make_rsrc(A.scale, BATCH * 4);
#pragma unroll
    for (int b = 0; b < BATCH; ++b) sclw[b] = __builtin_amdgcn_raw_buffer_load_b32(rscl, 4 * b, 0, 0);
  }
  // the replicated level table: a wave instruction writes four rows (16 lanes
  // x 16 bytes each); a lane takes the levels its row needs from lanes 0..15
  // with ds_bpermute
  {
    constexpr int kPerWave = (table_rows<IB>() / 4 + kWaves - 1) / kWaves;
    auto lv = [&](int i) { return (uint32_t)__builtin_amdgcn_ds_bpermute(i << 2, lv_lane); };
    uint4 ent[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int u = wave + i * kWaves;
      ent[i] = table_entry16<IB>(4 * u + (lane >> 4), lv);
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int u = wave + i * kWaves;
      if (u < table_rows<IB>() / 4)
        *reinterpret_cast<uint4 *>(tab + (4 * u + (lane >> 4)) * 256 + (lane & 15) * 16) = ent[i];
    }
  }
  // the first item goes out only now, so that the activations (every wave's
  // first loads) are not queued behind weight loads of other waves
  issue(ik, ipart, ring[0], nring[0]);
  advance(ik, ipart);
  // vmcnt(2 CPL): everything but the first item's loads has landed
  __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * CPL));

  // ---- 2. the rest of the ring, unconditionally
#pragma unroll
  for (int d = 1; d < PD; ++d) {
    issue(ik, ipart, ring[d], nring[d]);
    advance(ik, ipart);
  }

  // ---- 3. activations -> fp16 pairs in LDS
  if constexpr (FUSED) {
    const int spr = cols / kSeg;                   // segments per token
    float lmax[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) lmax[b] = 0.0f;
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg4 = (lane & 4) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      if (wave * kWave + j * kThreads >= nseg) continue;   // wave-uniform
      float *v = xv[j];
#pragma unroll
      for (int h = 1; h < kSeg; h <<= 1) {
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
          if ((i & h) == 0) {
            const float a = v[i], c = v[i + h];
            v[i] = a + c;
            v[i + h] = a - c;
          }
        }
      }
      // the stages across lanes (16, 32, 64, and 128 / 8 = 8 elements a
      // thread: stage 8 also): the partner element sits in lane ^ 1, ^ 2, ^ 4
      // (and ^ 8); the lower lane forms a + b, the upper one a - b (its own
      // value is b)
#pragma unroll
      for (int i = 0; i < kSeg; ++i) v[i] = fmaf(sg1, v[i], quad_xor1(v[i]));
#pragma unroll
      for (int i = 0; i < kSeg; ++i) v[i] = fmaf(sg2, v[i], quad_xor2(v[i]));
#pragma unroll
      for (int i = 0; i < kSeg; ++i) v[i] = fmaf(sg4, v[i], oct_xor4(v[i]));
      if constexpr (kSeg == 8) {
#pragma unroll
        for (int i = 0; i < kSeg; ++i) v[i] = fmaf(sg8, v[i], row_xor8(v[i]));
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < kSeg; ++i) m = fmaxf(m, fabsf(v[i]));
      const int bj = BATCH == 1 ? 0 : (t + j * kThreads) / spr;
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
        if (bj == b) lmax[b] = fmaxf(lmax[b], m);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const float mx = wave_max_to_lane63(lmax[b]);
      if (lane == 63) amax_red[b * kWaves + wave] = mx;
    }
    __syncthreads();
    // every wave forms the scales itself (same values, no second barrier)
    float scs[BATCH], invs[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      float mx = amax_red[b * kWaves];
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, amax_red[b * kWaves + w]);
      scs[b] = (mx > 0.0f) ? __fdiv_rn(mx, 127.0f) : 1.0f;
      invs[b] = __builtin_amdgcn_rcpf(scs[b]);
    }
    if (t < BATCH) s_blk[t] = scs[t];
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      const int sg = t + j * kThreads;
      if (sg < nseg) {
        const int b = BATCH == 1 ? 0 : sg / spr, k0 = (sg - b * spr) * kSeg;
        const int c = k0 >> 5, i0 = (k0 & 31) >> 3;     // chunk, and its (first) quarter
        float sc = scs[0], inv = invs[0];
#pragma unroll
        for (int bb = 1; bb < BATCH; ++bb)
          if (b == bb) { sc = scs[bb]; inv = invs[bb]; }
        // codes in blocks of 8 (bounded register use), packed to fp16 pairs
        uint32_t pr[8];
#pragma unroll
        for (int k8 = 0; k8 < kSeg / 8; ++k8) {
          float ub[8], cb[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) ub[i] = xv[j][8 * k8 + i];
          a8_codes<8>(ub, sc, inv, sc < 1.17549435e-38f, cb);
#pragma unroll
          for (int p = 0; p < 4; ++p)
            pr[4 * k8 + p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(cb[2 * p], cb[2 * p + 1]));
        }
        *reinterpret_cast<uint4 *>(&qs[((b * 4 + i0) * C + c) * 4]) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
        if constexpr (kSeg == 16)
          *reinterpret_cast<uint4 *>(&qs[((b * 4 + i0 + 1) * C + c) * 4]) = make_uint4(pr[4], pr[5], pr[6], pr[7]);
      }
    }
  } else {
    // 16 int8 codes a load: elements e0 .. e0+15 of token b = pairs p0 .. p0+7 of chunk c
#pragma unroll
    for (int j = 0; j < QV; ++j) {
      const int e0 = (t + j * kThreads) * 16;
      if (e0 < nq) {
        const int b = e0 / cols, k0 = e0 - b * cols;
        const int c = k0 >> 5, i0 = (k0 & 31) >> 3;     // quarter of the chunk: 0 or 2
        const uint32_t w4[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w};
        uint32_t pr[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t v = w4[h >> 1] >> (16 * (h & 1));
          h2 pp = {(_Float16)(int)(int8_t)v, (_Float16)(int)(int8_t)(v >> 8)};
          pr[h] = __builtin_bit_cast(uint32_t, pp);
        }
        *reinterpret_cast<uint4 *>(&qs[((b * 4 + i0) * C + c) * 4]) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
        *reinterpret_cast<uint4 *>(&qs[((b * 4 + i0 + 1) * C + c) * 4]) = make_uint4(pr[4], pr[5], pr[6], pr[7]);
      }
    }
  }
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
        const int c = li + P * (si * CPL + m);
        qpairs(b, c < C ? c : 0, qreg[b][m]);
        // chunks past the row's end: zero activations, so their (zero-index)
        // lookups add nothing whatever the norm
#pragma unroll
        for (int j = 0; j < 16; ++j) qreg[b][m][j] = c < C ? qreg[b][m][j] : 0u;
      }
  }

  // ---- 4. main loop
  float acc[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
  int pk = 0, ppart = 0;
  auto process = [&](Chunk<IB> (&cur)[CPL], const uint32_t (&ncur)[CPL]) {
    const int row = r0 + gw * rpw + rs + pk * rows_per_iter;
    const int sbase = (si * nparts + ppart) * CPL;
    // which half of the norm word: parity of the chunk's group index (for P = 64
    // the same for all CPL chunks: their groups differ by multiples of 16)
    const uint32_t nsh = (uint32_t)((row * ng + ((li + P * sbase) >> 2)) & 1) * 16u;
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
      const int c = li + P * (sbase + m);
      const bool cok = (FULL && QREG) || c < C;       // QREG: zero activations past the row
      const float nv = cok ? half_bits_to_float((uint16_t)(ncur[m] >> nsh)) : 0.0f;
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        uint32_t qq[16];
        if constexpr (QREG) {
#pragma unroll
          for (int j = 0; j < 16; ++j) qq[j] = qreg[b][m][j];
        } else {
          qpairs(b, cok ? c : 0, qq);
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
    if (ppart == nparts - 1) {           // uniform across the wave
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
      if (writer && row < r1) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) yblk[((row - r0) * S + si) * BATCH + b] = acc[b];
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
    }
    advance(pk, ppart);
  };
  for (int it0 = 0; it0 < NI; it0 += PD) {
#pragma unroll
    for (int d = 0; d < PD; ++d) {
      if (it0 + d < NI) process(ring[d], nring[d]);          // uniform branch, no memory ops
      issue(ik, ipart, ring[d], nring[d]);                   // refill: PD items ahead
      advance(ik, ipart);
    }
  }

  // ---- 5. rows out: the S partials of each row in a fixed order, coalesced
  __syncthreads();
  const int nr = r1 - r0;
  for (int i = t; i < nr * BATCH; i += kThreads) {
    const int b = i / nr, r = i - b * nr;
    float v = yblk[(r * S) * BATCH + b];
    for (int k = 1; k < S; ++k) v += yblk[(r * S + k) * BATCH + b];
    const float sc = FUSED ? s_blk[b] : __uint_as_float(sclw[b]);
    A.y[(size_t)b * rows + r0 + r] = v * (sc * (T.cscale * (1.0f / kGroup)));
  }
  if constexpr (FUSED) {
    // optional copies of the A8 result (block 0): codes back from the fp16 pairs
    if (blockIdx.x == 0) {
      if (A.scale_out && t < BATCH) A.scale_out[t] = s_blk[t];
      if (A.q_out) {
        for (int w = t; w < BATCH * cols / 4; w += kThreads) {
          const int b = (4 * w) / cols, k0 = 4 * w - b * cols;
          const int c = k0 >> 5, p = (k0 & 31) >> 1;        // pairs p, p + 1 of chunk c
          uint32_t out = 0;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const h2 pr = __builtin_bit_cast(h2, qs[((b * 4 + ((p + h) >> 2)) * C + c) * 4 + ((p + h) & 3)]);
            out |= ((uint32_t)(uint8_t)(int8_t)(int)(float)pr.x) << (16 * h);
            out |= ((uint32_t)(uint8_t)(int8_t)(int)(float)pr.y) << (16 * h + 8);
          }
          reinterpret_cast<uint32_t *>(A.q_out)[w] = out;
        }
      }
    }
  }
}

struct GemvConfig {
  int plog2, cpl, S, nparts;
  bool qreg;
};

// Lanes per row slot P (a power of two up to 64), chunks per lane per work
// item CPL (1, 2 or 4), parts per row NP and waves per row S, so that
// P * CPL * NP * S covers the row's C chunks.  Preferred: the smallest K split
// S that leaves a lane at most two chunks of a row (one work item per row, the
// activations in registers) while the rows still give every wave work.
// Measured on MI355X at the 8B-class decode shapes, this beats longer rows
// per wave (more parts, activations re-read from LDS) by 15-30%.
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
    if (S < 8 && slots > 2) continue;                     // long rows: split K further
    int cpl = slots <= 1 ? 1 : (slots <= 2 ? 2 : 4);
    if (cpl > max_cpl) cpl = max_cpl;
    cfg.plog2 = plog2;
    cfg.cpl = cpl;
    cfg.S = S;
    cfg.nparts = (slots + cpl - 1) / cpl;
    cfg.qreg = cfg.nparts == 1 && cpl * batch <= (cpl >= 4 ? 4 : 2);
    return true;
  }
  return false;
}

// Grid for a configuration: blocks, rows per block, and the work items every
// wave of a block walks (rows per block / rows per wave iteration x parts).
template <int CPL>
void grid_of(const bqm_cq_layout &L, const GemvConfig &cfg, int num_cus, int &blocks, int &rpb,
             int &items) {
  constexpr int kWaves = block_threads<CPL>() / kWave;
  const int rpw = kWave >> cfg.plog2;
  const int rows_per_iter = (kWaves / cfg.S) * rpw;
  blocks = (L.rows + rows_per_iter - 1) / rows_per_iter;
  if (blocks > num_cus) blocks = num_cus;
  rpb = (L.rows + blocks - 1) / blocks;             // rows per block (the tail iteration is partial)
  if (rpb * cfg.S > kMaxRowsBlk) rpb = kMaxRowsBlk / cfg.S;   // row partials fit in LDS
  blocks = (L.rows + rpb - 1) / rpb;
  items = (rpb + rows_per_iter - 1) / rows_per_iter * cfg.nparts;
}

template <int IB, int BATCH, int CPL, bool QREG, int PD, bool FUSED>
hipError_t launch_one(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      GemvArgs A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  constexpr int kThreads = block_threads<CPL>();
  int blocks, rpb, items;
  grid_of<CPL>(L, cfg, num_cus, blocks, rpb, items);
  const size_t qbytes = (size_t)BATCH * L.cols * 2;
  A.idx = blob;
  A.norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  A.rows = L.rows;
  A.cols = L.cols;
  A.plog2 = cfg.plog2;
  A.nparts = cfg.nparts;
  A.S = cfg.S;
  A.rows_per_block = rpb;
  A.idx_bytes = (uint32_t)L.idx_bytes;
  // whole 32-bit words: the norm words are read aligned, and the blob pads the
  // norms region to 64 bytes
  A.norm_bytes = (uint32_t)((L.norms_count * 2 + 3) & ~(int64_t)3);
  A.act_bytes = (uint32_t)((size_t)BATCH * L.cols * (FUSED ? 4 : 1));
  if constexpr (CPL == 1) {
    // rows shorter than 64 chunks: several rows per wave (only ever one chunk per lane)
    if (cfg.plog2 < 6) {
      cq_gemv_kernel<IB, BATCH, CPL, QREG, PD, false, FUSED, 16><<<blocks, kThreads, qbytes, s>>>(A, T);
      return hipGetLastError();
    }
  }
  // fused A8 of one token with more than 8192 columns: 8-element segments, two
  // a thread for most threads (measured faster there; slower at 4096 columns,
  // where one 16-element segment a thread keeps a quarter of the threads busy)
  if constexpr (FUSED && BATCH == 1 && CPL >= 2) {
    if (L.cols > 8192) {
      cq_gemv_kernel<IB, BATCH, CPL, QREG, PD, true, FUSED, 8><<<blocks, kThreads, qbytes, s>>>(A, T);
      return hipGetLastError();
    }
  }
  cq_gemv_kernel<IB, BATCH, CPL, QREG, PD, true, FUSED, 16><<<blocks, kThreads, qbytes, s>>>(A, T);
  return hipGetLastError();
}

// Work items in flight per wave: at most two (measured: deeper rings make every
// wave burst its loads up front, so its compute cannot start until the burst
// has drained; two items keep 64 KB per CU in flight and let a wave compute
// one item while the next streams), and at most kRingChunks chunks.
template <int BATCH, int CPL, bool FUSED>
constexpr int max_pd() {
  constexpr int kThreads = block_threads<CPL>();
  constexpr int kSeg = 16;                          // as in the kernel (KSEG 8: the same register count)
  constexpr int XREGS = FUSED ? (BATCH * kMaxFusedCols / kSeg + kThreads - 1) / kThreads * kSeg : 0;
  return (XREGS > 32 ? kRingChunks / 2 : kRingChunks) / CPL;
}

template <int IB, int BATCH, int CPL, bool QREG, bool FUSED>
hipError_t dispatch_pd(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                       const GemvArgs &A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  int blocks, rpb, items;
  grid_of<CPL>(L, cfg, num_cus, blocks, rpb, items);
  constexpr int kMax = max_pd<BATCH, CPL, FUSED>() < 2 ? max_pd<BATCH, CPL, FUSED>() : 2;
  if (items <= 1 || kMax == 1) return launch_one<IB, BATCH, CPL, QREG, 1, FUSED>(blob, L, T, A, cfg, num_cus, s);
  if constexpr (kMax >= 2) {
    if (items <= 2 || kMax == 2) return launch_one<IB, BATCH, CPL, QREG, 2, FUSED>(blob, L, T, A, cfg, num_cus, s);
  }
  if constexpr (kMax >= 4) {
    if (items <= 4 || kMax == 4) return launch_one<IB, BATCH, CPL, QREG, 4, FUSED>(blob, L, T, A, cfg, num_cus, s);
  }
  if constexpr (kMax >= 8) return launch_one<IB, BATCH, CPL, QREG, 8, FUSED>(blob, L, T, A, cfg, num_cus, s);
  return hipErrorInvalidValue;
}

template <int IB, int BATCH, int CPL, bool FUSED>
hipError_t dispatch_q(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                      const GemvArgs &A, const GemvConfig &cfg, int num_cus, hipStream_t s) {
  if constexpr (CPL * BATCH <= (CPL >= 4 ? 4 : 2)) {
    if (cfg.qreg) return dispatch_pd<IB, BATCH, CPL, true, FUSED>(blob, L, T, A, cfg, num_cus, s);
  }
  return dispatch_pd<IB, BATCH, CPL, false, FUSED>(blob, L, T, A, cfg, num_cus, s);
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
// fp16 copy of a launch's activations must fit in LDS beside the table.
template <int IB, bool FUSED>
hipError_t dispatch_batch(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, const float *x, int8_t *q_out,
                          float *scale_out, int batch, float *y, int num_cus, hipStream_t s) {
  const int C = L.cols / kChunk;
  for (int b0 = 0; b0 < batch;) {
    int nb = batch - b0 >= 4 ? 4 : (batch - b0 >= 2 ? 2 : 1);
    while (nb > 1 && (size_t)nb * L.cols * 2 > kMaxActLds) nb >>= 1;
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

// One instantiation set per (index bits, fused) lives in its own source file
// (cq_gemv_i<IB><f|q>.hip) so the build compiles them in parallel.
#define BQM_GEMV_VARIANT(IB, FUSED, NAME)                                                     \
  hipError_t NAME(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,          \
                  const int8_t *q, const float *scale, const float *x, int8_t *q_out,         \
                  float *scale_out, int batch, float *y, int num_cus, hipStream_t s) {        \
    return dispatch_batch<IB, FUSED>(blob, L, T, q, scale, x, q_out, scale_out, batch, y,    \
                                     num_cus, s);                                             \
  }

}  // namespace bqm
