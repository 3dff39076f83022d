// Base-3 ternary CQ weights (bits code 6) on the int8 matrix cores: batched
// decode (2..16 tokens a launch) and, 16 tokens a launch at a time, prefill.
//
// Format: the ternary CQ set of the Needle .cact/W4A8 article (section 1;
// levels {-c, 0, +c}), indices packed five to a byte as base-3 digits, the
// storage the llama.cpp TV-box / iPad page weighs against 2-bit fields (its
// speed-up table, section 18): a group of 128 is 26 bytes, byte j = sum_i
// idx[5j+i] * 3^i, digit 1 (the zero level) past the group's end.  The
// rotated-domain identity (article, section 3):
//   y[b, n] = s_b * c / 128 * sum_g norm[n, g] * sum_{k in g} (idx[n, k] - 1) * q[b, k]
// The inner sum is an exact integer (|.| <= 128 * 127), so it runs on
// v_mfma_i32_16x16x64_i8: A = 16 tokens x 64 k (the int8 codes), B = 64 k x 16
// weight rows (the digits minus one as int8), the int32 group sum scaled by
// the row's fp32 norm and added in fp32.
//
//  * Every weight byte takes 8 k slots: its five digits and three zeros, so a
//    byte's digits come from one 8-byte entry of an LDS table keyed by the
//    byte (entry v at v * 256 + (lane % 32) * 8: 32 copies, one per lane of a
//    half-wave, so a 64-bit read never shares a bank), one v_perm forming the
//    address.  A group's 26 bytes fill 208 of 256 slots: four MFMA steps.
//  * Lane (h, n) of a group supplies bytes 8 h .. 8 h + 7 of weight row n,
//    bytes 8 h + 2 s, 8 h + 2 s + 1 in step s; the A fragment of lane (h, t)
//    holds token t's codes of the same bytes' digits, 5 j .. 5 j + 4 of byte
//    j, each byte's three padding slots zero.  Bytes 26..31 of a group (past
//    its end: the next group's bytes, whatever they decode to) meet zero
//    codes, and so do the padding digits of byte 25.
//  * The rest follows the fp16 matrix-core GEMV: eight waves, one per eighth
//    of a K chunk of up to 32 groups; a wave converts its codes once into A
//    fragments kept in registers for all of the workgroup's 16-row blocks,
//    streams two blocks' weights in register rings, and the eighths meet in
//    LDS at the end.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads3 = 512;
constexpr int kWaves3 = kThreads3 / 64;    // one per eighth of K
constexpr int kTok3 = 16;                  // token rows of the MFMA tile
constexpr int kRBMax3 = 8;                 // 16-row blocks a workgroup finishes
constexpr int kChunk3 = 32;                // K chunk: groups whose codes the waves hold at once
constexpr int kMaxCols3 = 16384;
constexpr int kRings3 = 2;                 // row blocks whose weights are in flight at once
constexpr int kTab3 = 65536;               // digit table: 256 rows of 256 bytes
constexpr int kRed3 = kWaves3 * kRBMax3 * 4 * 64 * 4;   // partial sums [wave][block][r][lane]
static_assert(kTab3 + kRed3 <= 163840, "LDS of one CU");
constexpr uint32_t kOOB3 = 0x80000000u;
typedef int i32x4m __attribute__((ext_vector_type(4)));
typedef float f32x4m __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2m __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3m __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc3(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Table address of byte K of w: (byte << 8) | lo.
template <int K>
__device__ __forceinline__ uint32_t taddr3(uint32_t w, uint32_t lo) {
  return __builtin_amdgcn_perm(w, lo, 0x0C0C0000u | ((4u + K) << 8));
}

// The 8-byte table entry of byte value v: digit i of v minus one as int8 in
// byte i (i < 5), zeros in bytes 5..7; values past 242 are no digit string
// (all zero).
__device__ __forceinline__ uint2 digit_entry(uint32_t v) {
  if (v >= 243u) return make_uint2(0u, 0u);
  uint32_t b[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    b[i] = (uint32_t)(int32_t)((int)(v % 3u) - 1) & 0xFFu;
    v /= 3u;
  }
  return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4]);
}

// B operand of step s: the entries of the lane's bytes 2 s and 2 s + 1
// (bytes 0..3 in w0, 4..7 in w1).
template <int S>
__device__ __forceinline__ i32x4m digits_step(uint32_t w0, uint32_t w1, const uint8_t *tab, uint32_t lo) {
  const uint32_t w = S < 2 ? w0 : w1;
  constexpr int k0 = (S & 1) * 2;
  const uint2 a = *reinterpret_cast<const uint2 *>(tab + taddr3<k0>(w, lo));
  const uint2 b = *reinterpret_cast<const uint2 *>(tab + taddr3<k0 + 1>(w, lo));
  return i32x4m{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
}

// Bytes o .. o+3 and byte o of a run of dwords (o a compile-time byte offset).
template <int O>
__device__ __forceinline__ uint32_t get4(const uint32_t (&d)[10]) {
  if constexpr ((O & 3) == 0) return d[O >> 2];
  else return __builtin_amdgcn_alignbyte(d[(O >> 2) + 1], d[O >> 2], O & 3);
}
template <int O>
__device__ __forceinline__ uint32_t get1(const uint32_t (&d)[10]) {
  return (d[O >> 2] >> (8 * (O & 3))) & 0xFFu;
}

// The digit table, built by a workgroup of TH threads (512 or 1024): 16
// bytes a store, two copies of one entry.  Store i of thread t writes row
// v = t / 16 + (TH / 16) i; the wave's rows (4 wave + r + (TH / 16) i, r < 4)
// are computed once, by lane 4 i + r (and again by lane 32 + 4 i + r), and
// fetched from there with ds_bpermute.
template <int TH>
__device__ __forceinline__ void build_digit_table(uint8_t *tab, int t) {
  static_assert(kTab3 % (TH * 16) == 0 && kTab3 / (TH * 16) <= 8, "at most eight 16-byte stores a thread");
  constexpr int kStores = kTab3 / (TH * 16);
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6), lv = lane & 31;
  const uint2 mine = digit_entry((uint32_t)(4 * wave + (lv & 3) + (TH / 16) * (lv >> 2)));
#pragma unroll
  for (int i = 0; i < kStores; ++i) {
    const int src = (4 * i + (lane >> 4)) << 2;
    const uint32_t e0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mine.x);
    const uint32_t e1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mine.y);
    *reinterpret_cast<uint4 *>(tab + t * 16 + i * TH * 16) = make_uint4(e0, e1, e0, e1);
  }
}

struct T3MmaArgs {
  const uint8_t *blob;
  const uint16_t *norms;
  const int8_t *q;
  const float *scale;
  float *y;
  int rows, cols, batch;
  uint32_t blob_bytes, norm_bytes;
  float cfac;
};

// PD >= the groups of any eighth of a chunk; NRB row blocks of 16 rows per
// workgroup; CHUNKED: more than one chunk (the tiles (chunk, row block) then
// run in a loop whose weight loads run two tiles ahead, the next chunk's
// codes one chunk ahead, and the row blocks' partial sums gather in LDS).
template <int PD, int NRB, bool CHUNKED>
__global__ __launch_bounds__(kThreads3) void cq_t3_mma_kernel(T3MmaArgs A) {
  __shared__ __align__(16) uint8_t lds[kTab3 + kRed3];
  uint8_t *const tab = lds;
  float *const red = reinterpret_cast<float *>(lds + kTab3);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int K = A.cols, N = A.rows, ng = K / kGroup;
  const int nck = CHUNKED ? (ng + kChunk3 - 1) / kChunk3 : 1;
  const int ntiles = nck * NRB;
  const uint32_t row_bytes = (uint32_t)ng * kTritBytes;
  const int h = lane >> 4, l16 = lane & 15;
  const int rb0 = blockIdx.x * NRB;
  const __amdgpu_buffer_rsrc_t rw = rsrc3(A.blob, A.blob_bytes);
  const __amdgpu_buffer_rsrc_t rn = rsrc3(A.norms, A.norm_bytes);
  const __amdgpu_buffer_rsrc_t rq = rsrc3(A.q, (uint32_t)(A.batch * K));
  auto eighth = [&](int c, int &g0, int &ngw) {
    const int base = c * kChunk3;
    const int ngc = ng - base < kChunk3 ? ng - base : kChunk3;
    g0 = base + wave * ngc / kWaves3;
    ngw = base + (wave + 1) * ngc / kWaves3 - g0;
  };

  // codes of chunk c: lane (h, l16) takes token l16's codes 40 h .. 40 h + 39
  // of each group of the eighth (the digits of bytes 8 h .. 8 h + 7); codes
  // past the group's 128 read as zeros, and so do tokens past the batch
  // (16 + 16 + 8 bytes a group; lane h = 3 keeps only the first 8 of its
  // first 16, the rest being the next group's)
  typedef uint32_t Raw[PD][10];
  auto load_codes = [&](Raw &qraw, int c) {
    int g0, ngw;
    eighth(c, g0, ngw);
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int g = g0 + j < ng ? g0 + j : ng - 1;
      const uint32_t off = (uint32_t)(l16 * K + g * kGroup + 40 * h);
      const bool tail = h == 3;                    // codes 120 .. 127 only
      const u32x4m a0 = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      const u32x4m a1 = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rq, tail ? kOOB3 : off + 16u, 0, 0));
      const u32x2m a2 = __builtin_bit_cast(u32x2m, __builtin_amdgcn_raw_buffer_load_b64(
                                                       rq, tail ? kOOB3 : off + 32u, 0, 0));
      qraw[j][0] = a0.x; qraw[j][1] = a0.y;
      qraw[j][2] = tail ? 0u : a0.z; qraw[j][3] = tail ? 0u : a0.w;
      qraw[j][4] = a1.x; qraw[j][5] = a1.y; qraw[j][6] = a1.z; qraw[j][7] = a1.w;
      qraw[j][8] = a2.x; qraw[j][9] = a2.y;
    }
  };
  // as A fragments: step s holds bytes 2 s and 2 s + 1 of the lane's eight,
  // i.e. codes 10 s .. 10 s + 4 and 10 s + 5 .. 10 s + 9, each five followed
  // by three zeros
  i32x4m a[PD][4];
  auto convert = [&](const Raw &qraw) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      uint32_t d[10];
#pragma unroll
      for (int u = 0; u < 10; ++u) d[u] = qraw[j][u];
      a[j][0] = i32x4m{(int)get4<0>(d), (int)get1<4>(d), (int)get4<5>(d), (int)get1<9>(d)};
      a[j][1] = i32x4m{(int)get4<10>(d), (int)get1<14>(d), (int)get4<15>(d), (int)get1<19>(d)};
      a[j][2] = i32x4m{(int)get4<20>(d), (int)get1<24>(d), (int)get4<25>(d), (int)get1<29>(d)};
      a[j][3] = i32x4m{(int)get4<30>(d), (int)get1<34>(d), (int)get4<35>(d), (int)get1<39>(d)};
    }
  };

  // a ring: tile tt's weight bytes of the lane (row l16 of block rb0 + tt %
  // NRB, groups g0 + j of chunk tt / NRB: the 12 bytes from the 4-byte-aligned
  // address at or below byte 8 h of the group, realigned at use) and its
  // row's norms of the PD groups (the NW aligned words holding them, one load).
  // Past the matrix or the tiles the loads read zeros; past the eighth's
  // groups they read whatever lies there and the norm is taken as zero.
  typedef uint32_t Ring[PD][3];
  constexpr int NW = (PD + 2) / 2;
  typedef uint32_t NRing[NW];
  auto issue = [&](Ring &w, NRing &n, int tt) {
    int g0, ngw;
    eighth(tt / NRB, g0, ngw);
    const int row = (rb0 + tt % NRB) * 16 + l16;
    const bool ok = row < N && tt < ntiles;
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const uint32_t off = (uint32_t)row * row_bytes + (uint32_t)(g0 + j) * kTritBytes + 8u * h;
      const u32x3m v = __builtin_bit_cast(u32x3m, __builtin_amdgcn_raw_buffer_load_b96(rw, ok ? off & ~3u : kOOB3, 0, 2));
      w[j][0] = v.x; w[j][1] = v.y; w[j][2] = v.z;
    }
    // a word past the norm region (the region ends 64-byte aligned) reads 0
    const uint32_t nb = ok ? (((uint32_t)row * ng + g0) * 2u) & ~3u : kOOB3;
    if constexpr (NW == 3) {
      const u32x3m v = __builtin_bit_cast(u32x3m, __builtin_amdgcn_raw_buffer_load_b96(rn, nb, 0, 0));
      n[0] = v.x; n[1] = v.y; n[2] = v.z;
    } else if constexpr (NW == 2) {
      const u32x2m v = __builtin_bit_cast(u32x2m, __builtin_amdgcn_raw_buffer_load_b64(rn, nb, 0, 0));
      n[0] = v.x; n[1] = v.y;
    } else {
      n[0] = __builtin_amdgcn_raw_buffer_load_b32(rn, nb, 0, 0);
    }
  };

  const uint32_t lo = (uint32_t)(lane & 31) * 8u;
  // D[token][row] of tile tt: lane (h, l16) holds row l16, tokens 4 h + r
  auto consume = [&](const Ring &w, const NRing &n, int tt) {
    int g0, ngw;
    eighth(tt / NRB, g0, ngw);
    const int i = tt % NRB;
    const int row = (rb0 + i) * 16 + l16;
    // the norms' halves from group g0 on: the first sits in the high half of
    // word 0 when the row's norms start 2 bytes into a word
    const uint32_t p = ((uint32_t)row * ng + g0) & 1u;
    uint32_t nh[(PD + 1) / 2];
#pragma unroll
    for (int m = 0; m < (PD + 1) / 2; ++m)
      nh[m] = m + 1 < NW ? __builtin_amdgcn_alignbit(n[m + 1], n[m], p * 16u) : n[m] >> (p * 16u);
    f32x4m tot = f32x4m{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      // the group starts 2 bytes into its first dword when its byte offset is 2 mod 4
      const uint32_t sh = ((uint32_t)row * row_bytes + (uint32_t)(g0 + j) * kTritBytes) & 2u;
      const uint32_t w0 = __builtin_amdgcn_alignbyte(w[j][1], w[j][0], sh);
      const uint32_t w1 = __builtin_amdgcn_alignbyte(w[j][2], w[j][1], sh);
      i32x4m acc = i32x4m{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][0], digits_step<0>(w0, w1, tab, lo), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][1], digits_step<1>(w0, w1, tab, lo), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][2], digits_step<2>(w0, w1, tab, lo), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][3], digits_step<3>(w0, w1, tab, lo), acc, 0, 0, 0);
      const float nv = j < ngw ? half_bits_to_float((uint16_t)(nh[j >> 1] >> ((j & 1) * 16))) : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) tot[r] = fmaf(nv, (float)acc[r], tot[r]);
    }
    float *const slot = red + (wave * NRB + i) * 256 + lane;   // [r][lane]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (CHUNKED && tt >= NRB) tot[r] += slot[r * 64];
      slot[r * 64] = tot[r];
    }
  };

  constexpr int R = NRB < kRings3 && !CHUNKED ? NRB : kRings3;
  Raw qraw;
  load_codes(qraw, 0);
  Ring wr[R];
  NRing nr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) issue(wr[r], nr[r], r);

  build_digit_table<kThreads3>(tab, t);
  convert(qraw);
  if (CHUNKED) load_codes(qraw, 1);
  __syncthreads();

  if constexpr (!CHUNKED) {
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
  constexpr int wrows = NRB * 16;
  for (int e = t; e < kTok3 * wrows; e += kThreads3) {
    const int tk = e / wrows, rr = e - tk * wrows;
    const int i = rr >> 4, row16 = rr & 15;
    const int ln = 16 * (tk >> 2) + row16, r = tk & 3;
    float v = 0.0f;
#pragma unroll
    for (int w8 = 0; w8 < kWaves3; ++w8) v += red[((w8 * NRB + i) * 4 + r) * 64 + ln];
    const int row = blockIdx.x * wrows + rr;
    if (tk < A.batch && row < N) A.y[(size_t)tk * N + row] = v * (A.scale[tk] * A.cfac);
  }
}

// ------------------------------------------------------------------- GEMM
//
// Prefill: m tokens against the whole matrix, the weights read once per
// workgroup tile rather than once per 16 tokens.  v_mfma_i32_32x32x32_i8:
// A = 32 tokens x 32 k slots, B = 32 k slots x 32 weight rows, 16 slots (two
// weight bytes, five digits and three zeros each) a lane.  A group's 26 bytes
// and two more (past its end, meeting zero codes) are 7 steps of 4 bytes:
// lane half h takes bytes 14 h .. 14 h + 13, bytes 14 h + 2 s and + 1 in
// step s.  The int32 group sums are exact (|.| <= 128 * 127), scaled by the
// row's fp32 norm and added in fp32 once per group, in group order.
//  * Workgroup tile 64 MB tokens x 32 NB WN rows: 2 WN waves, two along the
//    tokens and WN along the rows, each 32 MB x 32 NB (MB x NB MFMA tiles).
//    Every wave runs all of K.
//  * The tokens' codes of one group are staged once per workgroup in LDS,
//    already laid out as A operands: per token 28 eight-byte slot groups (five
//    codes, three zeros; the codes past the group's 128 zero), 240 bytes a
//    token (an odd multiple of 16: the b128 fragment reads of 32 tokens fall
//    on distinct banks).  Two buffers: group g + 1 is staged while g is
//    multiplied, one barrier a group.
//  * Weights: a lane loads its row's 14 bytes of a group as the 20 bytes from
//    the 4-byte-aligned address below them (realigned with v_alignbyte),
//    two groups ahead, with the row's norm word.
constexpr int kT3GSlots = 28;              // slot groups (weight bytes) a group
constexpr int kT3GStride = 240;            // LDS bytes a token row of an A buffer
constexpr int kT3GSteps = 7;               // MFMA steps a group
typedef int i32x16m __attribute__((ext_vector_type(16)));

struct T3GemmArgs {
  const uint8_t *blob;
  const uint16_t *norms;
  const int8_t *q;
  const float *scale;
  float *y;
  int m, rows, cols, tiles_m, tiles_n;
  uint32_t blob_bytes, norm_bytes, q_bytes;
  float cfac;
};

template <int MB, int NB, int WN>
__global__ __launch_bounds__(128 * WN) void cq_t3_gemm_kernel(T3GemmArgs A) {
  constexpr int TH = 128 * WN;
  constexpr int BM = 64 * MB, BN = 32 * NB * WN;
  constexpr int kABuf = BM * kT3GStride;
  constexpr int kItems = BM * 7;                   // A staging items: 20 codes (4 slot groups) each
  constexpr int kIt = (kItems + TH - 1) / TH;
  static_assert(kTab3 + 2 * kABuf <= 163840, "LDS of one CU");
  __shared__ __align__(16) uint8_t lds[kTab3 + 2 * kABuf];
  uint8_t *const tab = lds;
  uint8_t *const abuf = lds + kTab3;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;

  // XCD-aware tile order: the m-tiles of one n-block (which share weights)
  // are consecutive tiles and run on one XCD
  const int ntiles = A.tiles_m * A.tiles_n;
  const int per = (ntiles + 7) / 8;
  const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (tile >= ntiles) return;
  const int mt = tile % A.tiles_m, nt = tile / A.tiles_m;
  const int m0 = mt * BM, n0 = nt * BN;
  const int K = A.cols, N = A.rows, ng = K / kGroup;
  const uint32_t row_bytes = (uint32_t)ng * kTritBytes;
  const __amdgpu_buffer_rsrc_t rw = rsrc3(A.blob, A.blob_bytes);
  const __amdgpu_buffer_rsrc_t rn = rsrc3(A.norms, A.norm_bytes);
  const __amdgpu_buffer_rsrc_t rq = rsrc3(A.q, A.q_bytes);

  // A staging: item i is token i / 7, codes 20 p .. 20 p + 19 (p = i % 7) of
  // the group, i.e. slot groups 4 p .. 4 p + 3; codes 128 .. 139 (p = 6,
  // dwords 2..4) are zero.  Rows past m and groups past K read zeros.
  uint32_t qoff[kIt];
  int iwhere[kIt];                                 // LDS byte offset of the item's 32 bytes, -1: none
  bool itail[kIt];
#pragma unroll
  for (int u = 0; u < kIt; ++u) {
    const int i = t + u * TH;
    const int tl = i / 7, p = i - 7 * (i / 7);
    const bool ok = i < kItems;
    iwhere[u] = ok ? tl * kT3GStride + 32 * p : -1;
    itail[u] = p == 6;
    qoff[u] = ok && m0 + tl < A.m ? (uint32_t)(m0 + tl) * (uint32_t)K + 20u * p : kOOB3;
  }
  uint32_t araw[kIt][5];
  auto load_a = [&](int g) {
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      const uint32_t off = g < ng && qoff[u] != kOOB3 ? qoff[u] + (uint32_t)g * kGroup : kOOB3;
      const u32x4m v = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      araw[u][0] = v.x; araw[u][1] = v.y; araw[u][2] = v.z; araw[u][3] = v.w;
      araw[u][4] = __builtin_amdgcn_raw_buffer_load_b32(rq, off + 16u, 0, 0);
    }
  };
  auto stage_a = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      if (iwhere[u] < 0) continue;
      const uint32_t d0 = araw[u][0], d1 = araw[u][1];
      const uint32_t d2 = itail[u] ? 0u : araw[u][2], d3 = itail[u] ? 0u : araw[u][3];
      const uint32_t d4 = itail[u] ? 0u : araw[u][4];
      const uint4 lo = make_uint4(d0, d1 & 0xFFu, __builtin_amdgcn_alignbyte(d2, d1, 1), (d2 >> 8) & 0xFFu);
      const uint4 hi = make_uint4(__builtin_amdgcn_alignbyte(d3, d2, 2), (d3 >> 16) & 0xFFu,
                                  __builtin_amdgcn_alignbyte(d4, d3, 3), d4 >> 24);
      uint8_t *dst = abuf + buf * kABuf + iwhere[u];
      *reinterpret_cast<uint4 *>(dst) = lo;
      *reinterpret_cast<uint4 *>(dst + 16) = hi;
    }
  };

  // B: row n = n0 + 32 (NB wn + nb) + lr of each n-block nb; its 14 bytes of
  // group g from 26 g + 14 lh, and the word holding its norm
  uint32_t wbase[NB], nidx[NB];
  bool nok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + 32 * (NB * wn + nb) + lr;
    nok[nb] = n < N;
    wbase[nb] = (uint32_t)n * row_bytes + 14u * lh;
    nidx[nb] = (uint32_t)n * (uint32_t)ng;
  }
  uint32_t wraw[2][NB][5], nraw[2][NB];
  auto load_b = [&](int g, int slot) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool ok = nok[nb] && g < ng;
      const uint32_t off = ok ? (wbase[nb] + (uint32_t)g * kTritBytes) & ~3u : kOOB3;
      const u32x4m v = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
      wraw[slot][nb][0] = v.x; wraw[slot][nb][1] = v.y; wraw[slot][nb][2] = v.z; wraw[slot][nb][3] = v.w;
      wraw[slot][nb][4] = __builtin_amdgcn_raw_buffer_load_b32(rw, off + 16u, 0, 0);
      nraw[slot][nb] = __builtin_amdgcn_raw_buffer_load_b32(rn, ok ? ((nidx[nb] + (uint32_t)g) * 2u) & ~3u : kOOB3, 0, 0);
    }
  };

  float tot[MB][NB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[mb][nb][r] = 0.0f;

  const uint32_t lo = (uint32_t)lr * 8u;
  // lane's A fragment rows: tokens 32 (MB wm + mb) + lr, slot groups 14 lh + 2 s, + 1
  const int afrag = (32 * MB * wm + lr) * kT3GStride + 112 * lh;
  auto mult = [&](int g, int slot) {
    uint32_t wd[NB][4];
    float nv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t sh = (wbase[nb] + (uint32_t)g * kTritBytes) & 2u;
#pragma unroll
      for (int e = 0; e < 4; ++e) wd[nb][e] = __builtin_amdgcn_alignbyte(wraw[slot][nb][e + 1], wraw[slot][nb][e], sh);
      nv[nb] = half_bits_to_float((uint16_t)(nraw[slot][nb] >> (((nidx[nb] + (uint32_t)g) & 1u) * 16u)));
    }
    const uint8_t *ab = abuf + (g & 1) * kABuf + afrag;
    i32x16m acc[MB][NB];
#pragma unroll
    for (int s = 0; s < kT3GSteps; ++s) {
      i32x4m af[MB], bf[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const i32x4m *>(ab + 32 * mb * kT3GStride + 16 * s);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t w = wd[nb][s >> 1];
        const uint2 e0 = *reinterpret_cast<const uint2 *>(tab + ((s & 1) ? taddr3<2>(w, lo) : taddr3<0>(w, lo)));
        const uint2 e1 = *reinterpret_cast<const uint2 *>(tab + ((s & 1) ? taddr3<3>(w, lo) : taddr3<1>(w, lo)));
        bf[nb] = i32x4m{(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              af[mb], bf[nb], s == 0 ? i32x16m{} : acc[mb][nb], 0, 0, 0);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tot[mb][nb][r] = fmaf(nv[nb], (float)acc[mb][nb][r], tot[mb][nb][r]);
  };

  load_a(0);
  load_b(0, 0);
  load_b(1, 1);
  build_digit_table<TH>(tab, t);
  stage_a(0);
  load_a(1);
  __syncthreads();
  // group g: stage g + 1 (its codes loaded during g - 1), load the codes of
  // g + 2, multiply g, load the weights of g + 2 into g's ring slot
  for (int g0 = 0; g0 < ng; g0 += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int g = g0 + d;
      if (g < ng) {
        stage_a((g + 1) & 1);
        load_a(g + 2);
        mult(g, d);
        load_b(g + 2, d);
      }
      __syncthreads();
    }
  }

  // D layout: register r of a lane holds token 8 (r / 4) + 4 lh + r % 4,
  // row lr of its 32 x 32 tile
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * (MB * wm + mb) + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (m >= A.m) continue;
      const float f = A.scale[m] * A.cfac;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = n0 + 32 * (NB * wn + nb) + lr;
        if (n < N) A.y[(size_t)m * N + n] = tot[mb][nb][r] * f;
      }
    }
}

template <int MB, int NB, int WN>
hipError_t launch_t3_gemm_tiles(T3GemmArgs A, hipStream_t s) {
  A.tiles_m = (A.m + 64 * MB - 1) / (64 * MB);
  A.tiles_n = (A.rows + 32 * NB * WN - 1) / (32 * NB * WN);
  const int grid = ((A.tiles_m * A.tiles_n + 7) / 8) * 8;
  cq_t3_gemm_kernel<MB, NB, WN><<<grid, 128 * WN, 0, s>>>(A);
  return hipGetLastError();
}

}  // namespace

bool cq_t3_mma_supported(const bqm_cq_layout &L, int batch) {
  return batch >= 2 && batch <= kTok3 && L.group == kGroup && L.cols % kGroup == 0 &&
         L.cols <= kMaxCols3 && L.total_bytes < ((int64_t)1 << 31);
}

hipError_t launch_cq_t3_mma(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                            const int8_t *q, const float *scale, int batch, float *y, int num_cus,
                            hipStream_t s) {
  const int rb_total = (L.rows + 15) / 16;
  const int per_cu = (rb_total + num_cus - 1) / num_cus;
  const int nrb = per_cu <= 1 ? 1 : per_cu <= 2 ? 2 : per_cu <= 4 ? 4 : kRBMax3;
  const int grid = (rb_total + nrb - 1) / nrb;
  T3MmaArgs A{};
  A.blob = blob;
  A.norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  A.q = q;
  A.scale = scale;
  A.y = y;
  A.rows = L.rows;
  A.cols = L.cols;
  A.batch = batch;
  // the whole blob: a lane's 12-byte window of a row's last group reaches
  // past the index region into the norms (or the 64-byte padding after them)
  A.blob_bytes = (uint32_t)L.total_bytes;
  A.norm_bytes = (uint32_t)(L.total_bytes - L.norms_offset);   // whole words (64-byte padded)
  A.cfac = T.cscale / (float)kGroup;
  const int ng = L.cols / kGroup, pd_need = (ng + kWaves3 - 1) / kWaves3;
  auto with_nrb = [&](auto pd, auto chunked) -> hipError_t {
    constexpr int PD = decltype(pd)::value;
    constexpr bool CH = decltype(chunked)::value;
    switch (nrb) {
      case 1: cq_t3_mma_kernel<PD, 1, CH><<<grid, kThreads3, 0, s>>>(A); break;
      case 2: cq_t3_mma_kernel<PD, 2, CH><<<grid, kThreads3, 0, s>>>(A); break;
      case 4: cq_t3_mma_kernel<PD, 4, CH><<<grid, kThreads3, 0, s>>>(A); break;
      default: cq_t3_mma_kernel<PD, kRBMax3, CH><<<grid, kThreads3, 0, s>>>(A); break;
    }
    return hipGetLastError();
  };
  if (ng > kChunk3) return with_nrb(std::integral_constant<int, 4>{}, std::true_type{});
  if (pd_need > 2) return with_nrb(std::integral_constant<int, 4>{}, std::false_type{});
  if (pd_need > 1) return with_nrb(std::integral_constant<int, 2>{}, std::false_type{});
  return with_nrb(std::integral_constant<int, 1>{}, std::false_type{});
}

bool cq_t3_gemm_supported(const bqm_cq_layout &L, int m) {
  return m >= 1 && L.group == kGroup && L.cols % kGroup == 0 && L.total_bytes < ((int64_t)1 << 31) &&
         (int64_t)m * L.cols < ((int64_t)1 << 31) - 64;
}

// Tile shape: the largest of 128 x 256, 128 x 128, 64 x 128 (tokens x rows)
// whose tile count still covers 7/8 of the CUs, else 64 x 128.
hipError_t launch_cq_t3_gemm(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                             const int8_t *q, const float *scale, int m, float *y, int num_cus,
                             hipStream_t s) {
  T3GemmArgs A{};
  A.blob = blob;
  A.norms = reinterpret_cast<const uint16_t *>(blob + L.norms_offset);
  A.q = q;
  A.scale = scale;
  A.y = y;
  A.m = m;
  A.rows = L.rows;
  A.cols = L.cols;
  A.blob_bytes = (uint32_t)L.total_bytes;                     // windows past a row's end stay in the blob
  A.norm_bytes = (uint32_t)(L.total_bytes - L.norms_offset);   // whole words (64-byte padded)
  A.q_bytes = (uint32_t)((int64_t)m * L.cols);
  A.cfac = T.cscale / (float)kGroup;
  auto tiles = [&](int bm, int bn) { return (long)((m + bm - 1) / bm) * ((L.rows + bn - 1) / bn); };
  // the largest tile that covers 7/8 of the CUs in one round; one round of
  // larger tiles on at least half the CUs beats two rounds of smaller ones
  const long want = (long)num_cus * 7 / 8;
  const long t256 = tiles(128, 256), t128 = tiles(128, 128), t64 = tiles(64, 128);
  if (t256 >= want || (t128 > num_cus && 2 * t256 >= num_cus)) return launch_t3_gemm_tiles<2, 1, 8>(A, s);
  if (t128 >= want || (t64 > num_cus && 2 * t128 >= num_cus)) return launch_t3_gemm_tiles<2, 1, 4>(A, s);
  return launch_t3_gemm_tiles<1, 1, 4>(A, s);
}

}  // namespace bqm
