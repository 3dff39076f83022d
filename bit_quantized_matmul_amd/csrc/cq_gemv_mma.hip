// Batched decode GEMV (2..32 tokens) on packed CQ weights, on the matrix cores.
//
// "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
// quantization", section 3: decode streams the pre-transposed [out, in] rows
// once per call, and section 1 fixes the group-128 codebook + fp16-norm
// format.  The sum is the GEMV's, for up to 16 tokens at once:
//   y[b, n] = scale[b] * cscale / 128 * sum_g norm[n, g] * sum_{k in g} lv[idx[n, k]] * q[b, k]
//
// Past a few tokens the per-token dot products, not the weight stream, bound a
// VALU GEMV.  Here one pass over the weights serves every token:
//  * v_mfma_f32_16x16x32_f16 with A = 16 tokens x 32 k (the int8 codes as exact
//    fp16) and B = 32 k x 16 weight rows (levels looked up from a replicated
//    LDS table, exact in fp16).  Products are exact and accumulate in fp32; a
//    lane of the 16x16 result holds one weight row, so each group's result is
//    scaled by that row's fp32 norm (no rounding of level x norm, unlike the
//    prefill GEMM).
//  * In a group a lane supplies the 32 contiguous indices 32 h .. 32 h + 31 of
//    its row (h = lane / 16): step s feeds k = 32 h + 8 s .. + 8 to the MFMA's
//    k slice 8 h .. 8 h + 8.  A and B use the same order, so the sum is the
//    group's, and a lane's weight bytes for a group are one contiguous load.
//  * Eight waves per workgroup, one per eighth of K.  A wave converts the 16
//    tokens' codes of its eighth once into A fragments it keeps in registers
//    for every 16-row block of the workgroup (1, 2, 4 or 8 blocks, fixed per
//    kernel so the code is straight-line), and holds two blocks' weights in
//    register rings, the next block's loads going out as a block is used
//    (more in flight only delays the first block behind the queued loads).
//  * The eighths of a row block meet once, through LDS, at the end.
//  * 17..32 tokens (cq_gemm's few-token calls): two 16-token halves, each
//    looked-up B fragment feeding one MFMA per half; the K chunk and the row
//    blocks a workgroup takes are halved to make room for the second half's
//    A fragments and partial sums.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreadsV = 512;
constexpr int kWaves = kThreadsV / 64;  // one per eighth of K
constexpr int kTok = 16;                // token columns of the MFMA tile
constexpr int kMaxTok = 2 * kTok;       // tokens a launch takes (two 16-token halves)
constexpr int kRBMax = 8;               // row blocks a workgroup finishes
constexpr int kChunkGroups = 32;        // K chunk: the groups whose codes the waves hold at once
// With two token halves (TH = 2) a wave holds twice the A fragments and
// partial sums: past one chunk of 32 groups (where the next chunk's codes are
// in flight too) the K chunk is halved, and so are the row blocks a workgroup
// takes.
template <int TH> constexpr int chunk_groups() { return kChunkGroups / TH; }
template <int TH> constexpr int rb_max() { return kRBMax / TH; }
constexpr int kMaxCols = 16384;         // as the fused GEMV's limit
constexpr int kMaxRings = 2;            // row blocks whose weights are in flight at once
constexpr int kTabBytes = 65536;        // level table: 256-byte rows
// partial sums [wave][block][half][r][lane]
template <int NRB, int TH> constexpr int red_bytes() { return kWaves * NRB * TH * 4 * 64 * 4; }
static_assert(kTabBytes + red_bytes<kRBMax, 1>() <= 163840 && kTabBytes + red_bytes<rb_max<2>(), 2>() <= 163840,
              "LDS of one CU");
constexpr uint32_t kOOBv = 0x80000000u;
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS serves a 64-lane read in parts that each cover its 64 banks (256 bytes)
// once: all 64 lanes of a 4-byte read, 32 of an 8-byte one, 16 of a 16-byte
// one.  Every table row is 256 bytes, entry e of `eb` bytes replicated across
// it and lane l reading its copy at e * 256 + (l * eb) % 256, so the lanes of
// a part never share a bank, and one v_perm turns an index byte into the
// address.  Entries: an index byte's levels (8 for 1-bit indices, 4 for 2-bit,
// 2 for 4-bit), or a 6-bit pair of 3-bit indices.
template <int IB> constexpr int entry_b() { return IB == 1 ? 16 : (IB == 2 ? 8 : 4); }
template <int IB> constexpr int tab_rows() { return IB == 3 ? 64 : 256; }

// fp16 bits of level i, picked from the levels held in scalar registers (no
// memory access: the table build waits on nothing in flight)
template <int NL>
__device__ __forceinline__ uint32_t level_bits(const LevelTable &T, uint32_t i) {
  uint32_t v[NL];
#pragma unroll
  for (int c = 0; c < NL; ++c) v[c] = T.h16[c];
#pragma unroll
  for (int w = NL / 2; w >= 1; w /= 2)
#pragma unroll
    for (int c = 0; c < w; ++c) v[c] = (i & (uint32_t)w) ? v[c + w] : v[c];
  return v[0];
}

// 16 bytes of table row e (its entry, replicated).  Lane c < 16 of `lv` holds
// level c's fp16 bits; 3- and 4-bit indices gather their levels from there,
// smaller sets select among their few levels directly.
template <int IB>
__device__ __forceinline__ uint4 entry16(int e, const LevelTable &T, uint32_t lv) {
  if constexpr (IB == 4 || IB == 3) {
    constexpr int m = (1 << IB) - 1;
    const uint32_t a = (uint32_t)__builtin_amdgcn_ds_bpermute((e & m) << 2, (int)lv);
    const uint32_t b = (uint32_t)__builtin_amdgcn_ds_bpermute((e >> IB) << 2, (int)lv);
    const uint32_t v = a | (b << 16);
    return make_uint4(v, v, v, v);
  } else if constexpr (IB == 2) {
    const uint32_t a = level_bits<4>(T, e & 3) | (level_bits<4>(T, (e >> 2) & 3) << 16);
    const uint32_t b = level_bits<4>(T, (e >> 4) & 3) | (level_bits<4>(T, (e >> 6) & 3) << 16);
    return make_uint4(a, b, a, b);
  } else {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = level_bits<2>(T, (e >> (2 * j)) & 1) | (level_bits<2>(T, (e >> (2 * j + 1)) & 1) << 16);
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// Table address of index byte K of w: v_perm forms (byte << 8) | lo.
template <int K>
__device__ __forceinline__ uint32_t taddr(uint32_t w, uint32_t lo) {
  return __builtin_amdgcn_perm(w, lo, 0x0C0C0000u | ((4u + K) << 8));
}

// B operand of step s (0..3): the levels of indices 8 s .. 8 s + 7 of the
// lane's 32, whose codes sit in IB words.
template <int IB>
__device__ __forceinline__ f16x8v levels_step(const uint32_t (&wd)[IB], int s, const uint8_t *tab, uint32_t lo) {
  uint32_t r[4];
  if constexpr (IB == 4) {
    const uint32_t w = wd[s];
    r[0] = *reinterpret_cast<const uint32_t *>(tab + taddr<0>(w, lo));
    r[1] = *reinterpret_cast<const uint32_t *>(tab + taddr<1>(w, lo));
    r[2] = *reinterpret_cast<const uint32_t *>(tab + taddr<2>(w, lo));
    r[3] = *reinterpret_cast<const uint32_t *>(tab + taddr<3>(w, lo));
  } else if constexpr (IB == 2) {
    const uint32_t w = wd[s >> 1];
    uint2 e0, e1;
    if (s & 1) {
      e0 = *reinterpret_cast<const uint2 *>(tab + taddr<2>(w, lo));
      e1 = *reinterpret_cast<const uint2 *>(tab + taddr<3>(w, lo));
    } else {
      e0 = *reinterpret_cast<const uint2 *>(tab + taddr<0>(w, lo));
      e1 = *reinterpret_cast<const uint2 *>(tab + taddr<1>(w, lo));
    }
    r[0] = e0.x; r[1] = e0.y; r[2] = e1.x; r[3] = e1.y;
  } else if constexpr (IB == 1) {
    const uint32_t w = wd[0];
    uint4 e;
    switch (s & 3) {
      case 0: e = *reinterpret_cast<const uint4 *>(tab + taddr<0>(w, lo)); break;
      case 1: e = *reinterpret_cast<const uint4 *>(tab + taddr<1>(w, lo)); break;
      case 2: e = *reinterpret_cast<const uint4 *>(tab + taddr<2>(w, lo)); break;
      default: e = *reinterpret_cast<const uint4 *>(tab + taddr<3>(w, lo)); break;
    }
    r[0] = e.x; r[1] = e.y; r[2] = e.z; r[3] = e.w;
  } else {                                   // IB == 3: 24 bits = four 6-bit pair fields
    const int bit = 24 * s;
    const int wi = bit >> 5, sh = bit & 31;
    const uint32_t lw = wd[wi];
    const uint32_t hw = (wi + 1 < IB) ? wd[wi + 1] : 0u;
    const uint32_t v = __builtin_amdgcn_alignbit(hw, lw, sh);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t f = __builtin_amdgcn_ubfe(v, 6 * p, 6);
      r[p] = *reinterpret_cast<const uint32_t *>(tab + ((f << 8) | lo));
    }
  }
  f16x8v out;
  __builtin_memcpy(&out, r, 16);
  return out;
}

// IB consecutive words at byte `off` (streamed: non-temporal)
template <int IB>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[IB]) {
  if constexpr (IB == 4) {
    const u32x4v a = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else if constexpr (IB == 3) {
    const u32x3v a = __builtin_bit_cast(u32x3v, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 2));
    w[0] = a.x; w[1] = a.y; w[2] = a.z;
  } else if constexpr (IB == 2) {
    const u32x2v a = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
    w[0] = a.x; w[1] = a.y;
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2);
  }
}

// int8 x4 -> four fp16 (exact): bits 0x6400 | (q + 128) equal 1152 + q.
__device__ __forceinline__ void i8x4_f16(uint32_t w, uint32_t &lo, uint32_t &hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - bias);
}

struct MmaArgs {
  const uint8_t *idx;
  const uint16_t *norms;
  const int8_t *q;
  const float *scale;
  float *y;
  int rows, cols, batch;
  uint32_t idx_bytes, norm_bytes;
};

// K is taken in chunks of up to kChunkGroups groups (cols <= kChunkGroups *
// 128 is one chunk).  PD >= the groups of any eighth of a chunk; NRB row
// blocks of 16 rows per workgroup; CHUNKED: more than one chunk, the tiles
// (chunk, row block) then run in a loop whose weight loads run two tiles
// ahead across chunk ends, the next chunk's codes one chunk ahead, and the
// row blocks' partial sums gather in LDS.  KS = 2: workgroups 2 j and 2 j + 1
// take the two halves of K of the same row blocks, each reading only its
// half's codes, and add their results into y, which the caller has zeroed:
// two addends onto zero give the same sum in either order.  TH: token halves
// (1: up to 16 tokens; 2: up to 32, each B fragment feeding one MFMA per half).
template <int IB, int PD, int NRB, bool CHUNKED, int KS, int TH>
__global__ __launch_bounds__(kThreadsV) void cq_gemv_mma_kernel(MmaArgs A, LevelTable T) {
  constexpr int kCG = CHUNKED ? chunk_groups<TH>() : kChunkGroups;
  // one array, the table at its start: table addresses need no base added
  __shared__ __align__(16) uint8_t lds[kTabBytes + red_bytes<NRB, TH>()];
  uint8_t *const tab = lds;
  float *const red = reinterpret_cast<float *>(lds + kTabBytes);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // the eighth of each chunk
  const int K = A.cols, N = A.rows, ng = K / kGroup;
  const int kh = KS == 1 ? 0 : (int)blockIdx.x % KS;           // this workgroup's part of K
  const int rg = KS == 1 ? (int)blockIdx.x : (int)blockIdx.x / KS;
  const int gb = kh * ng / KS, ge = (kh + 1) * ng / KS;       // its groups gb .. ge - 1
  const int nck = CHUNKED ? (ge - gb + kCG - 1) / kCG : 1;
  const int ntiles = nck * NRB;
  const int row_bytes = K * IB / 8;
  const int h = lane >> 4, l16 = lane & 15;
  const int rb0 = rg * NRB;
  const __amdgpu_buffer_rsrc_t ridx = rsrc(A.idx, A.idx_bytes);
  const __amdgpu_buffer_rsrc_t rnrm = rsrc(A.norms, A.norm_bytes);
  const __amdgpu_buffer_rsrc_t rq = rsrc(A.q, (uint32_t)(A.batch * K));
  // the wave's groups of chunk c: g0 .. g0 + ngw - 1 (ngw <= PD)
  auto eighth = [&](int c, int &g0, int &ngw) {
    const int base = gb + c * kCG;
    const int ngc = ge - base < kCG ? ge - base : kCG;
    g0 = base + wave * ngc / kWaves;
    ngw = base + (wave + 1) * ngc / kWaves - g0;
  };

  // codes of chunk c: lane (h, l16) takes token 16 th + l16's codes 32 h ..
  // 32 h + 31 of each group of the eighth (tokens past the batch read as
  // zeros; slots past the eighth repeat a group in range, their norm is taken
  // as zero)
  typedef u32x4v Raw[TH][PD][2];
  auto load_codes = [&](Raw &qraw, int c) {
    int g0, ngw;
    eighth(c, g0, ngw);
#pragma unroll
    for (int th = 0; th < TH; ++th)
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        const int g = g0 + j < ng ? g0 + j : ng - 1;
        const uint32_t off = (uint32_t)((16 * th + l16) * K + g * kGroup + 32 * h);
        qraw[th][j][0] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        qraw[th][j][1] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0));
      }
  };
  // as fp16 A fragments: step s takes codes 8 s .. 8 s + 7
  f16x8v a[TH][PD][4];
  auto convert = [&](const Raw &qraw) {
#pragma unroll
    for (int th = 0; th < TH; ++th)
#pragma unroll
      for (int j = 0; j < PD; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4v &v = qraw[th][j][s >> 1];
          uint32_t o[4];
          i8x4_f16((s & 1) ? v.z : v.x, o[0], o[1]);
          i8x4_f16((s & 1) ? v.w : v.y, o[2], o[3]);
          __builtin_memcpy(&a[th][j][s], o, 16);
        }
  };

  // a ring: tile tt's weight words of the lane and its row's norms (row l16
  // of block rb0 + tt % NRB, groups g0 + j of chunk tt / NRB), the norms as
  // the NW aligned words that hold them.  Past the matrix or the tiles the
  // loads read zeros; past the eighth's groups they read whatever lies there
  // and the norm is taken as zero.
  constexpr int NW = (PD + 2) / 2;
  typedef uint32_t Ring[PD][IB];
  typedef uint32_t NRing[NW];
  auto issue = [&](Ring &w, NRing &n, int tt) {
    int g0, ngw;
    eighth(tt / NRB, g0, ngw);
    const int row = (rb0 + tt % NRB) * 16 + l16;
    const bool ok = row < N && tt < ntiles;
    const uint32_t wbase = ok ? (uint32_t)(row * row_bytes + g0 * (16 * IB) + h * (4 * IB)) : kOOBv;
    const uint32_t nbase = ok ? (uint32_t)(row * ng + g0) * 2u : kOOBv;
#pragma unroll
    for (int j = 0; j < PD; ++j) load_words<IB>(ridx, wbase + (uint32_t)(j * 16 * IB), w[j]);
    load_words<NW>(rnrm, nbase & ~3u, n);
  };

  const uint32_t lo = (uint32_t)(lane * entry_b<IB>()) & 255u;
  // D[token][row] of tile tt: lane (h, l16) holds row l16, tokens
  // 16 th + 4 h + r; added into the row block's partial sums
  auto consume = [&](const Ring &w, const NRing &n, int tt) {
    int g0, ngw;
    eighth(tt / NRB, g0, ngw);
    const int i = tt % NRB;
    // the norms' halves from group g0 on: the first sits in the high half
    // of word 0 when the row's norms start 2 bytes into a word
    const uint32_t p = (uint32_t)(((rb0 + i) * 16 + l16) * ng + g0) & 1u;
    uint32_t nh[(PD + 1) / 2];
#pragma unroll
    for (int m = 0; m < (PD + 1) / 2; ++m)
      nh[m] = m + 1 < NW ? __builtin_amdgcn_alignbit(n[m + 1], n[m], p * 16u) : n[m] >> (p * 16u);
    f32x4v tot[TH];
#pragma unroll
    for (int th = 0; th < TH; ++th) tot[th] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      f32x4v acc[TH];
#pragma unroll
      for (int th = 0; th < TH; ++th) acc[th] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8v b = levels_step<IB>(w[j], s, tab, lo);
#pragma unroll
        for (int th = 0; th < TH; ++th)
          acc[th] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[th][j][s], b, acc[th], 0, 0, 0);
      }
      const float nv = j < ngw ? half_bits_to_float((uint16_t)(nh[j >> 1] >> ((j & 1) * 16))) : 0.0f;
#pragma unroll
      for (int th = 0; th < TH; ++th)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[th][r] = fmaf(nv, acc[th][r], tot[th][r]);
    }
#pragma unroll
    for (int th = 0; th < TH; ++th) {
      float *const slot = red + ((wave * NRB + i) * TH + th) * 256 + lane;   // [r][lane]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (CHUNKED && tt >= NRB) tot[th][r] += slot[r * 64];
        slot[r * 64] = tot[th][r];
      }
    }
  };

  constexpr int R = NRB < kMaxRings && !CHUNKED ? NRB : kMaxRings;
  Raw qraw;
  load_codes(qraw, 0);
  Ring wr[R];
  NRing nr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) issue(wr[r], nr[r], r);

  // level table: lanes 0 .. 15 hold the levels' fp16 bits, gathered from
  // there by the 3- and 4-bit entries
  uint32_t lv = 0;
  if constexpr (IB >= 3) {
#pragma unroll
    for (int c = 0; c < (1 << IB); ++c) lv = lane == c ? (uint32_t)T.h16[c] : lv;
  }
#pragma unroll
  for (int o = t * 16; o < tab_rows<IB>() * 256; o += kThreadsV * 16)
    *reinterpret_cast<uint4 *>(tab + o) = entry16<IB>(o >> 8, T, lv);
  convert(qraw);
  if (CHUNKED) load_codes(qraw, 1);
  __syncthreads();

  if constexpr (!CHUNKED) {
    // row block i in ring i % R; once a ring is used, block i + R's loads go
    // into it (kept in place against the scheduler, which would sink them)
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      consume(wr[i % R], nr[i % R], i);
      if (i + R < NRB) {
        __builtin_amdgcn_sched_barrier(0);
        issue(wr[i % R], nr[i % R], i + R);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // tiles in pairs, tile tt in ring tt % 2; at a chunk's first tile its
    // codes (loaded a chunk ago) become the A fragments and the next chunk's
    // codes are requested
    for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int tt = t0 + r;
        if (tt < ntiles) {
          if (tt > 0 && tt % NRB == 0) {
            convert(qraw);
            load_codes(qraw, tt / NRB + 1 < nck ? tt / NRB + 1 : nck - 1);
          }
          consume(wr[r], nr[r], tt);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(wr[r], nr[r], tt + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // the eighths of each row block, in a fixed order
  __syncthreads();
  const float cfac = T.cscale * (1.0f / kGroup);
  constexpr int wrows = NRB * 16;              // the workgroup's rows, per token
  for (int e = t; e < kTok * TH * wrows; e += kThreadsV) {
    const int tk = e / wrows, rr = e - tk * wrows;
    const int i = rr >> 4, row16 = rr & 15;
    const int th = tk >> 4, t16 = tk & 15;
    const int ln = 16 * (t16 >> 2) + row16, r = t16 & 3;
    float v = 0.0f;
#pragma unroll
    for (int w8 = 0; w8 < kWaves; ++w8) v += red[(((w8 * NRB + i) * TH + th) * 4 + r) * 64 + ln];
    const int row = rg * wrows + rr;
    if (tk < A.batch && row < N) {
      if constexpr (KS == 1) A.y[(size_t)tk * N + row] = v * (A.scale[tk] * cfac);
      else atomicAdd(&A.y[(size_t)tk * N + row], v * (A.scale[tk] * cfac));
    }
  }
}

__global__ void zero_f32_kernel(float *__restrict__ y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0.0f;
}

}  // namespace

bool cq_gemv_mma_supported(const bqm_cq_layout &L, int batch) {
  // 2 tokens only where K is one chunk: with chunks the VALU GEMV, which
  // holds no codes, is as fast for 2
  const int min_batch = L.cols <= kChunkGroups * kGroup ? 2 : 3;
  return batch >= min_batch && batch <= kMaxTok && L.cols % kGroup == 0 && L.cols <= kMaxCols &&
         (uint64_t)L.idx_bytes < (1u << 30) && (uint64_t)L.norms_count * 2 < (1u << 30);
}

namespace {

template <int TH>
hipError_t launch_mma_th(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                         const int8_t *q, const float *scale, int batch, float *y,
                         int num_cus, hipStream_t s) {
  constexpr int kCG = chunk_groups<TH>(), kRB = rb_max<TH>();   // (kCG: when chunked)
  // a workgroup per CU where that leaves each at most kRB row blocks, the
  // count rounded up to a power of two
  const int rb_total = (L.rows + 15) / 16;
  const int per_cu = (rb_total + num_cus - 1) / num_cus;
  const int ng = L.cols / kGroup, pd_need = (ng + kWaves - 1) / kWaves;
  // one row block a CU, long rows and more than 8 tokens (the codes a
  // workgroup reads then outweigh its weights): split K in two (each
  // workgroup two row blocks, half the codes), the halves added into y after
  // a zero fill (the fill's launch costs as much as the split saves at 4 tokens)
  const bool split = per_cu <= 1 && ng >= 2 * kChunkGroups && rb_total >= 2 && batch > 8;
  const int nrb = split ? 2 : per_cu <= 1 ? 1 : per_cu <= 2 ? 2 : per_cu <= 4 || kRB == 4 ? 4 : kRB;
  const int grid = (rb_total + nrb - 1) / nrb * (split ? 2 : 1);
  if (split) {
    const int n = batch * L.rows;
    zero_f32_kernel<<<(n + 255) / 256, 256, 0, s>>>(y, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  MmaArgs A{};
  A.idx = blob;
  A.norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  A.q = q;
  A.scale = scale;
  A.y = y;
  A.rows = L.rows;
  A.cols = L.cols;
  A.batch = batch;
  A.idx_bytes = (uint32_t)L.idx_bytes;
  A.norm_bytes = (uint32_t)((L.norms_count * 2 + 3) & ~(int64_t)3);
  auto with_nrb = [&](auto ib, auto pd, auto chunked) -> hipError_t {
    constexpr int IB = decltype(ib)::value, PD = decltype(pd)::value;
    constexpr bool CH = decltype(chunked)::value;
    if (CH && split) {
      cq_gemv_mma_kernel<IB, PD, 2, CH, 2, TH><<<grid, kThreadsV, 0, s>>>(A, T);
      return hipGetLastError();
    }
    switch (nrb) {
      case 1: cq_gemv_mma_kernel<IB, PD, 1, CH, 1, TH><<<grid, kThreadsV, 0, s>>>(A, T); break;
      case 2: cq_gemv_mma_kernel<IB, PD, 2, CH, 1, TH><<<grid, kThreadsV, 0, s>>>(A, T); break;
      case 4: cq_gemv_mma_kernel<IB, PD, 4, CH, 1, TH><<<grid, kThreadsV, 0, s>>>(A, T); break;
      default: cq_gemv_mma_kernel<IB, PD, kRB, CH, 1, TH><<<grid, kThreadsV, 0, s>>>(A, T); break;
    }
    return hipGetLastError();
  };
  auto go = [&](auto ib) -> hipError_t {
    constexpr int kPDC = kCG / kWaves;             // groups of an eighth of a full chunk
    if (ng > kChunkGroups)
      return with_nrb(ib, std::integral_constant<int, kPDC>{}, std::true_type{});
    if (pd_need > 2) return with_nrb(ib, std::integral_constant<int, 4>{}, std::false_type{});
    if (pd_need > 1) return with_nrb(ib, std::integral_constant<int, 2>{}, std::false_type{});
    return with_nrb(ib, std::integral_constant<int, 1>{}, std::false_type{});
  };
  switch (L.index_bits) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 3: return go(std::integral_constant<int, 3>{});
    default: return go(std::integral_constant<int, 4>{});
  }
}

}  // namespace

hipError_t launch_cq_gemv_mma(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                              const int8_t *q, const float *scale, int batch, float *y,
                              int num_cus, hipStream_t s) {
  if (batch > kTok) return launch_mma_th<2>(blob, L, T, q, scale, batch, y, num_cus, s);
  return launch_mma_th<1>(blob, L, T, q, scale, batch, y, num_cus, s);
}

}  // namespace bqm
