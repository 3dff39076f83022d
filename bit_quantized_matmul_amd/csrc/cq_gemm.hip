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
//    bank-conflict-free table as the GEMV), and scales each fp16 level pair by
//    the group's norm times 2^e_n with one packed fp16 multiply.  e_n is an
//    exponent per weight row n, chosen from the row's largest norm so that
//    level x norm x 2^e_n stays below 2^15 for every level and group of the
//    row; norm x 2^e_n is formed exactly with one v_ldexp_f16.  The packed
//    multiply is then the one rounding of the path: at most
//    2^-11 relative per weight for every group whose products stay in fp16's
//    normal range, i.e. whose norm is at least ~2^-23 of the row's largest
//    (smaller groups round to fp16 subnormals, an absolute error below
//    2^-39 of the row's largest level x norm per weight).  MFMA products of
//    fp16 operands are exact and accumulate in fp32
//    (v_mfma_f32_32x32x16_f16) straight through all of K: no per-group
//    epilogue interrupts the chain.  The epilogue multiplies each column by
//    2^-e_n, exactly.
//  * The k order inside a group is permuted consistently for A and B: in step
//    s (0..7) lane half h supplies columns 64h + 8s .. +8, so each lane reads
//    one contiguous run of 64 indices per group.
//  * Eight waves per workgroup, two per SIMD, so one wave's LDS and barrier
//    waits overlap the other's MFMAs.  Waves 0-3 take steps 0-3 of every
//    group and waves 4-7 steps 4-7 (a split of K inside the workgroup, summed
//    once at the end through LDS); within a half the four waves form a
//    WM x (4 / WM) grid of MB x NB MFMA tiles of 32 x 32 each.  A wave's LDS
//    reads per step are MB A fragments and NB level lookups, and its VALU
//    work (address perms, norm multiplies) scales with NB alone, so the
//    tiles use tall waves side by side: 128 x 64 each in the wide tile,
//    128 x 32 in the 128 x 128 one and 64 x 32 in the 64 x 128 one (2 x 2
//    grids of 64 x 64 and 32 x 64 waves spent ~7 and ~11.5 VALU instructions
//    per MFMA there, against ~5 and ~7).  The launch takes the largest
//    workgroup tile that still gives every CU work (128 x 256 for wide
//    matrices, 128 x 128, or 64 x 128).  Consecutive tiles (the m-tiles of one
//    n-block, which share weights) are mapped to the same XCD: hardware deals
//    workgroups round-robin over the 8 XCDs.
//  * Norms: a wave's norm load touches one cache line per row (32 per
//    instruction) for 2 bytes each, as costly as an index load.  When the
//    group count is a multiple of 8 (K a multiple of 1024), a row's norms for
//    8 consecutive groups are one aligned 16-byte load, made a round of 8
//    groups ahead into a second register set; otherwise every group loads its
//    own.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads = 512;                 // 8 waves: two per SIMD
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

// B operand for step s (0..3) of a lane's half group: the 8 levels of indices
// 8s .. 8s+7 of its 32, whose codes sit in IB words (4*IB bytes).
template <int IB, int NW>
__device__ __forceinline__ f16x8 lookup_step(const uint32_t (&wd)[NW], int s,
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
    const uint32_t w = wd[0];
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
    const uint32_t hi = (wi + 1 < IB) ? wd[wi + 1] : 0u;
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
constexpr uint32_t kOOB = 0x80000000u;     // buffer offset past every range: reads give 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// The lane's index bytes of one group for its steps (8 indices a step): NW
// whole words (IB words for half a group's steps, IB / 2 for a quarter).
template <int NW>
__device__ __forceinline__ void load_b_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else if constexpr (NW == 3) {
    const u32x3 a = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0));
    w[0] = a.x; w[1] = a.y; w[2] = a.z;
  } else if constexpr (NW == 2) {
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    w[0] = a.x; w[1] = a.y;
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}

// Loads run kDepth groups ahead in registers through raw buffer loads (rows
// past M or N read zeros), all issued unconditionally so the compiler waits
// for exactly one group's loads at a time; groups past K read zeros too, so
// the loop runs a whole number of rounds with no branch.  N8: the group count
// is a multiple of 8 and norms come 8 groups to a load.  KS: the split of
// each group's 8 steps over the workgroup's waves (2: halves, four waves a
// half; 4: quarters, two waves a quarter, for the narrow 64 x 32 tile).
template <int IB, int WM, int MB, int NB, bool N8, int KS>
__global__ __launch_bounds__(kThreads) void cq_gemm_kernel(
    const uint8_t *__restrict__ idx, const uint16_t *__restrict__ norms,
    const int8_t *__restrict__ q, const float *__restrict__ scale, float *__restrict__ y,
    int M, int N, int K, int tiles_m, int tiles_n, uint32_t idx_bytes, uint32_t norm_bytes,
    LevelTable T) {
  constexpr int TB = table_bytes<IB>();
  constexpr int kDepth = N8 ? 4 : 3;               // groups of A and B in flight per thread
  constexpr int kRound = N8 ? 8 : kDepth;          // groups per loop round (unrolled)
  constexpr int kWPK = 8 / KS;                     // waves per k slice
  constexpr int kSteps = 8 / KS;                   // 16-wide k steps of a wave per group
  constexpr int kBW = kSteps * IB / 4;             // index words of a lane per group
  constexpr int WN = kWPK / WM;
  constexpr int kBM = 32 * MB * WM, kBN = 32 * NB * WN;
  static_assert((KS == 2 || KS == 4) && kBW * 4 == kSteps * IB && WM * WN == kWPK,
                "whole index words per lane and group; the waves of a slice tile it");
  constexpr int kAV = kBM / 64;                    // 16-byte A loads per thread per group
  constexpr int kYS = kBN + 8;                     // epilogue tile row stride (floats): rows 4 apart sit 32 banks apart
  constexpr int kLoopBytes = TB + 2 * kBM * kAStride * 2, kYBytes = kBM * kYS * 4;
  static_assert(kThreads == 512 && kGroup == 128 && kAV >= 1, "A staging: 8 lanes per 128-byte row slice, 64 rows a pass");
  // One LDS array: the level table at offset 0 (a lookup address is the
  // v_perm result itself, no base add) and two A buffers; the epilogue then
  // reuses it for the fp32 output tile.
  __shared__ __align__(16) uint8_t smem[kLoopBytes > kYBytes ? kLoopBytes : kYBytes];
  uint8_t *const tab = smem;
  _Float16 (*As)[kBM * kAStride] = reinterpret_cast<_Float16 (*)[kBM * kAStride]>(smem + TB);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int kq = wave / kWPK;                      // which KS-th of each group's 8 steps
  const int wm = (wave % kWPK) / WN, wn = (wave % kWPK) % WN;
  const int lr = lane & 31, lh = lane >> 5;

  // XCD-aware tile order: tiles xcd*per .. xcd*per+per-1 run on one XCD
  const int ntiles = tiles_m * tiles_n;
  const int per = (ntiles + 7) / 8;
  const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (tile >= ntiles) return;
  const int mt = tile % tiles_m, nt = tile / tiles_m;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int ng = K / kGroup;
  const int rounds = (ng + kRound - 1) / kRound;
  const int row_bytes = K * IB / 8;
  const uint32_t laneoff = (uint32_t)(lane * entry_bytes<IB>()) & 255u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(q, (uint32_t)((size_t)M * K));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(idx, idx_bytes);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(norms, norm_bytes);

  for (int o = t * 16; o < TB; o += kThreads * 16)
    *reinterpret_cast<uint4 *>(tab + o) = table_entry16<IB>(o >> 8, T);

  // A: load i of thread t is 16 int8 of row t / 8 + 64 i at bytes 16 (t % 8) of
  // the group, so eight lanes read one row's whole 128-byte slice
  const int arow0 = t >> 3, acol = (t & 7) * 16;
  uint32_t abase[kAV];
#pragma unroll
  for (int i = 0; i < kAV; ++i) {
    const int r = m0 + arow0 + 64 * i;
    abase[i] = r < M ? (uint32_t)(r * K + acol) : kOOB;
  }
  // B: per n-block nb, lane holds row n = n0 + 32 NB wn + 32 nb + lr; of the
  // group's 8*IB-byte run of indices 64 lh .. 64 lh + 63 it loads the half its
  // steps use (4*IB bytes)
  int ncol[NB];
  uint32_t bbase[NB], nbase[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    ncol[nb] = n0 + 32 * NB * wn + 32 * nb + lr;
    const bool ok = ncol[nb] < N;
    bbase[nb] = ok ? (uint32_t)(ncol[nb] * row_bytes + 8 * IB * lh + kSteps * IB * kq) : kOOB;
    nbase[nb] = ok ? (uint32_t)(ncol[nb] * ng * 2) : kOOB;
  }
  // The row exponents: each lane needs e_n for its NB rows.  The two lanes of
  // a wave that supply row n (lane halves lh = 0, 1) read alternate pieces of
  // the row's norms (16-byte pieces of 8 norms when the group count is a
  // multiple of 8, else single norms) and combine their maxima.  Norms are
  // non-negative, so their fp16 bit patterns order as their values.  The
  // first batch of loads (up to 64 groups a row) is issued here, before the
  // main loads, and reduced after them; longer rows finish in a loop.
  constexpr int kPre = 4;                          // pre-pass loads per row and batch
  constexpr int kPerLoad = N8 ? 8 : 1;             // norms per pre-pass load
  const int pieces = N8 ? ng / 8 : ng;
  uint32_t pre[kPre][NB][N8 ? 4 : 1];
  auto issue_pre = [&](int j0) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int j = j0 + 2 * u;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t off = j < pieces ? nbase[nb] + (uint32_t)(2 * kPerLoad * j) : kOOB;
        if constexpr (N8) {
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, off, 0, 0));
          pre[u][nb][0] = v.x; pre[u][nb][1] = v.y; pre[u][nb][2] = v.z; pre[u][nb][3] = v.w;
        } else {
          pre[u][nb][0] = __builtin_amdgcn_raw_buffer_load_b16(rn, off, 0, 0);
        }
      }
    }
  };
  uint32_t nmax[NB];
  auto reduce_pre = [&]() {
#pragma unroll
    for (int u = 0; u < kPre; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < (N8 ? 4 : 1); ++i) {
          const uint32_t w = pre[u][nb][i];
          nmax[nb] = max(nmax[nb], max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
        }
  };
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) nmax[nb] = 0;
  issue_pre(lh);

  // Each n-block walks the groups from its own starting point (wrapping), so
  // the n-blocks that share A rows read different k-slices at any one time
  // instead of all hitting the same memory channels together.  The m-tiles of
  // one n-block (on one XCD) walk in step: they read each weight group at
  // about the same time, and all but the first find it in L2.  (N8: a
  // multiple of 8, so every round's 8 groups share one aligned norm load.)
  const int rot = N8 ? ((nt * 7) % (ng / 8)) * 8 : (nt * 7) % ng;
  // Loop steps past the last group (the loop runs whole rounds)
  // reload group 0 with a zero norm scale, so they add exact zeros and every
  // load stays unconditional (no branch, no early vmcnt drain).
  auto kgroup = [&](int g) { const int x = g + rot; return g >= ng ? 0 : (x < ng ? x : x - ng); };
  u32x4 apre[kDepth][kAV];
  uint32_t bpre[kDepth][NB][kBW], npre[N8 ? 1 : kDepth][NB];
  u32x4 ncur[NB], nnext[NB];                       // N8: norms of this loop round's groups and the next one's
  auto issue_norms = [&](int g0, u32x4 (&dst)[NB]) {
    const int gg = kgroup(g0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      dst[nb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, nbase[nb] + 2u * gg, 0, 0));
  };
  auto issue = [&](int g, int slot) {
    const int gg = kgroup(g);
#pragma unroll
    for (int i = 0; i < kAV; ++i)
      apre[slot][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          ra, abase[i] + (uint32_t)(gg * kGroup), 0, 0));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      load_b_words<kBW>(rb, bbase[nb] + (uint32_t)(gg * 16 * IB), bpre[slot][nb]);
      if constexpr (!N8)
        npre[slot][nb] = __builtin_amdgcn_raw_buffer_load_b32(rn, (nbase[nb] + 2u * gg) & ~3u, 0, 0);
    }
  };
  // one 16-byte A load (16 int8) -> 16 fp16 in LDS buffer buf
  auto store_a_part = [&](int slot, int buf, int i) {
    _Float16 *dst = &As[buf][(arow0 + 64 * i) * kAStride + acol];
    uint32_t o[8];
    i8x4_to_f16x4(apre[slot][i].x, o[0], o[1]);
    i8x4_to_f16x4(apre[slot][i].y, o[2], o[3]);
    i8x4_to_f16x4(apre[slot][i].z, o[4], o[5]);
    i8x4_to_f16x4(apre[slot][i].w, o[6], o[7]);
    *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4 *>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if constexpr (N8) issue_norms(0, ncur);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(d, d);
  // the rest of the row exponents' pre-pass (the first batch has landed by
  // the time the first A stores wait for their loads)
  reduce_pre();
  for (int j0 = 2 * kPre; j0 < pieces; j0 += 2 * kPre) {   // a trip count the wave shares
    issue_pre(j0 + lh);
    reduce_pre();
  }
  // e_n = fold_exp - E_M with E_M = floor(log2(largest norm)): then
  // norm x 2^e_n < 2^15 and level x norm x 2^e_n < 2^15 for every level
  // (fold_exp = 13 - max(floor(log2(largest |level|)), -1), from the host)
  int rexp[NB];                                    // e_n
  float rinv[NB];                                  // 2^-e_n
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t hm = max(nmax[nb], (uint32_t)__shfl_xor((int)nmax[nb], 32, 64));
    int e;
    if (hm == 0) e = 0;                            // an all-zero row (or a row past N)
    else if (hm >= 0x7C00u) e = -2;                // inf / NaN norms: no scaling can help
    else if (hm >= 0x400u) e = T.fold_exp - ((int)(hm >> 10) - 15);
    else e = T.fold_exp - ((31 - __builtin_clz(hm)) - 24);   // subnormal largest norm
    rexp[nb] = e;
    rinv[nb] = __uint_as_float((uint32_t)(127 - e) << 23);
  }

#pragma unroll
  for (int i = 0; i < kAV; ++i) store_a_part(0, 0, i);
  __syncthreads();

  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  // A wave's half group runs as 4 steps x MB chunks; chunk (s, mb) is the NB
  // MFMAs of m-block mb at step s.  Around them the wave issues the work of
  // later chunks, in a fixed order that the scheduling barriers keep: the A
  // fragment two chunks ahead, the next step's level lookups (at mb 0) and
  // norm multiplies (at the last mb), a part of the next group's A staging.
  // The last step looks up the next group's first step (the table never
  // changes); the workgroup barrier sits in the last chunk, where every wave
  // has written its part of the next group's A and read its last fragment of
  // this group's, followed by the next group's first A reads.
  constexpr int kChunks = kSteps * MB;
  h2v nq[NB];
  f16x8 lvr[NB], bfr[2][NB], ar[3];
  auto scale_b = [&](const f16x8 &lv, h2v f) {
    f16x8 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const h2v rr = h2v{lv[2 * p], lv[2 * p + 1]} * f;
      o[2 * p] = rr.x;
      o[2 * p + 1] = rr.y;
    }
    return o;
  };
  // group g's norm x 2^e_n as an fp16 pair (v_ldexp_f16: exact, since the
  // result is at most 2^15 and, but for groups far below the row's largest,
  // normal; groups past K get 2^-64, i.e. zero): from
  // prefetch slot d, or (N8) from this loop round's or the next one's norms,
  // where group g is halfword g % 8
  auto take_group = [&](int g, int d, bool next) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t nw;
      if constexpr (N8) {
        const u32x4 v = next ? nnext[nb] : ncur[nb];
        const int hw = g & 7;
        nw = v[hw >> 1] >> ((hw & 1) * 16);
      } else {
        nw = npre[d][nb] >> ((((uint32_t)(ncol[nb] * ng + kgroup(g))) & 1u) * 16u);
      }
      const _Float16 h = __builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)nw), g < ng ? rexp[nb] : -64);
      nq[nb] = h2v{h, h};
    }
  };
  // lane's A fragment for chunk c: rows 32 (MB wm + mb) + lr, step kSteps kq + s
  const int afrag = (32 * MB * wm + lr) * kAStride + 64 * lh + 8 * kSteps * kq;
  auto read_a = [&](int buf, int c) {
    return *reinterpret_cast<const f16x8 *>(&As[buf][afrag + 32 * (c % MB) * kAStride + 8 * (c / MB)]);
  };
  take_group(0, 0, false);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) lvr[nb] = lookup_step<IB, kBW>(bpre[0][nb], 0, tab, laneoff);
  ar[0] = read_a(0, 0);
  if (kChunks > 1) ar[1] = read_a(0, 1);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) bfr[0][nb] = scale_b(lvr[nb], nq[nb]);
  __builtin_amdgcn_sched_barrier(0);
  for (int r0 = 0; r0 < rounds; ++r0) {
#pragma unroll
    for (int d8 = 0; d8 < kRound; ++d8) {
      const int g = r0 * kRound + d8;
      const int d = d8 % kDepth;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int s = c / MB, mb = c % MB;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ar[c % 3], bfr[s & 1][nb], acc[mb][nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (mb == 0) {
          const bool last = s == kSteps - 1;
          const int sl = last ? (d + 1) % kDepth : d;   // the last step looks up the next group
          if (last) take_group(g + 1, sl, d8 == kRound - 1);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            lvr[nb] = lookup_step<IB, kBW>(bpre[sl][nb], last ? 0 : s + 1, tab, laneoff);
        }
        if (c + 2 < kChunks) ar[(c + 2) % 3] = read_a(g & 1, c + 2);
        if (c >= 1 && c <= kAV) store_a_part((d + 1) % kDepth, (g + 1) & 1, c - 1);   // A of group g + 1
        if (mb == MB - 1) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) bfr[(s + 1) & 1][nb] = scale_b(lvr[nb], nq[nb]);
        }
        if (c == kChunks - 1) {
          issue(g + kDepth, d);                    // refill this slot, kDepth groups ahead
          if (N8 && d8 == 0) issue_norms(g + kRound, nnext);
          __syncthreads();
          ar[0] = read_a((g + 1) & 1, 0);
          if (kChunks > 1) ar[1] = read_a((g + 1) & 1, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (N8) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ncur[nb] = nnext[nb];
    }
  }

  // Epilogue through LDS (free now).  The KS k-slices meet there in a fixed
  // order: the waves of the last slice park their accumulators as an fp32
  // tile, those of each earlier slice in turn add theirs in place; then each
  // row leaves as whole 16-byte chunks, so one store instruction writes a run
  // of contiguous bytes.  MFMA D layout: register r of a lane holds row
  // 8 (r / 4) + 4 lh + r % 4, column lr of its 32 x 32 tile.
  float *const ys = reinterpret_cast<float *>(smem);
  auto ypos = [&](int mb, int nb, int r) {
    return (32 * MB * wm + 32 * mb + 8 * (r >> 2) + 4 * lh + (r & 3)) * kYS + 32 * NB * wn + 32 * nb + lr;
  };
  __syncthreads();                                 // every wave is done with the table and A buffers
  // (column lr of tile nb is weight row ncol[nb]: its 2^-e_n is exact)
#pragma unroll
  for (int j = KS - 1; j >= 0; --j) {
    if (kq == j) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int p = ypos(mb, nb, r);
            const float v = acc[mb][nb][r] * rinv[nb];
            ys[p] = j == KS - 1 ? v : v + ys[p];
          }
    }
    __syncthreads();
  }
  const float cfac = T.cscale * (1.0f / kGroup);
  constexpr int kLPR = kBN / 4;                    // threads per tile row, 4 columns each
  constexpr int kRPP = kThreads / kLPR;            // rows per pass
  const int cr = t / kLPR, cc = (t % kLPR) * 4;
  const int n = n0 + cc;
  const bool vec = ((N & 3) == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
#pragma unroll 4
  for (int p = 0; p < kBM / kRPP; ++p) {
    const int row = p * kRPP + cr, m = m0 + row;
    if (m >= M) continue;
    const float f = scale[m] * cfac;
    const float4 v = *reinterpret_cast<const float4 *>(&ys[row * kYS + cc]);
    float *dst = y + (size_t)m * N + n;
    if (vec && n + 3 < N) {
      *reinterpret_cast<float4 *>(dst) = make_float4(v.x * f, v.y * f, v.z * f, v.w * f);
    } else {
      if (n < N) dst[0] = v.x * f;
      if (n + 1 < N) dst[1] = v.y * f;
      if (n + 2 < N) dst[2] = v.z * f;
      if (n + 3 < N) dst[3] = v.w * f;
    }
  }
}

template <int IB, int WM, int MB, int NB, int KS = 2>
hipError_t launch_tiles(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                        const int8_t *q, const float *scale, int m, float *y, hipStream_t s) {
  constexpr int kBM = 32 * MB * WM, kBN = 32 * NB * (8 / KS / WM);
  const int tiles_m = (m + kBM - 1) / kBM;
  const int tiles_n = (L.rows + kBN - 1) / kBN;
  const int grid = ((tiles_m * tiles_n + 7) / 8) * 8;
  const uint16_t *norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  const uint32_t ib = (uint32_t)L.idx_bytes;
  const uint32_t nbytes = (uint32_t)((L.norms_count * 2 + 3) & ~(int64_t)3);   // whole words (blob pads to 64)
  if ((L.cols / kGroup) % 8 == 0)
    cq_gemm_kernel<IB, WM, MB, NB, true, KS><<<grid, kThreads, 0, s>>>(blob, norms, q, scale, y, m, L.rows, L.cols,
                                                                   tiles_m, tiles_n, ib, nbytes, T);
  else
    cq_gemm_kernel<IB, WM, MB, NB, false, KS><<<grid, kThreads, 0, s>>>(blob, norms, q, scale, y, m, L.rows, L.cols,
                                                                    tiles_m, tiles_n, ib, nbytes, T);
  return hipGetLastError();
}

// Tile shape: the largest of 128x256, 128x128, 64x128 (m x n) whose tile count
// still covers the CUs in one round, else 64x64, or 64x32 where even 64x64
// leaves CUs idle (few tokens or rows: the launch is a weight stream and wants
// every CU on it).  One round of larger tiles on at
// least half the CUs beats two rounds of smaller ones (512 x 11008 x 4096:
// 71 us in 172 tiles of 128 x 256 against 87 us in 344 of 128 x 128).
template <int IB>
hipError_t launch_ib(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                     const int8_t *q, const float *scale, int m, float *y, int num_cus,
                     hipStream_t s) {
  auto tiles = [&](int bm, int bn) {
    return (long)((m + bm - 1) / bm) * ((L.rows + bn - 1) / bn);
  };
  const long full = (long)num_cus * 7 / 8;
  const long t256 = tiles(128, 256), t128 = tiles(128, 128), t64 = tiles(64, 128);
  if (t256 >= full || (t128 > num_cus && 2 * t256 >= num_cus))
    return launch_tiles<IB, 1, 4, 2>(blob, L, T, q, scale, m, y, s);
  if (t128 >= full || (t64 > num_cus && 2 * t128 >= num_cus))
    return launch_tiles<IB, 1, 4, 1>(blob, L, T, q, scale, m, y, s);
  if (t64 >= full)
    return launch_tiles<IB, 1, 2, 1>(blob, L, T, q, scale, m, y, s);
  // fewer than 7/8 of the CUs with 64 x 64 tiles: 64 x 32 tiles (each group's
  // steps in quarters, two 32 x 32 waves a quarter), twice the workgroups
  // (measured: 512 x 1024 x 4096 20.5 against 22.7-23.8 us, 64 x 4096 x 4096
  // 19.4 against 21.9, 32 x 4096 x 14336 53.5 against 64.7)
  if constexpr (IB == 2 || IB == 4)
    if (tiles(64, 64) < full) return launch_tiles<IB, 2, 1, 1, 4>(blob, L, T, q, scale, m, y, s);
  return launch_tiles<IB, 2, 1, 1>(blob, L, T, q, scale, m, y, s);
}

}  // namespace

hipError_t launch_cq_gemm(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int m, float *y, int num_cus,
                          hipStream_t s) {
  switch (L.index_bits) {
    case 1: return launch_ib<1>(blob, L, T, q, scale, m, y, num_cus, s);
    case 2: return launch_ib<2>(blob, L, T, q, scale, m, y, num_cus, s);
    case 3: return launch_ib<3>(blob, L, T, q, scale, m, y, num_cus, s);
    default: return launch_ib<4>(blob, L, T, q, scale, m, y, num_cus, s);
  }
}

}  // namespace bqm
