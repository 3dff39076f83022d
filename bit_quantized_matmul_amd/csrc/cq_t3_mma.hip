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

  // the digit table: 16 bytes a store, two copies of one entry.  Store i of
  // thread t writes row v = t / 16 + 32 i; the wave's 32 rows (4 wave + r +
  // 32 i, r < 4) are computed once, by lane 4 i + r (and again by lane
  // 32 + 4 i + r), and fetched from there with ds_bpermute.
  static_assert(kTab3 == 8 * kThreads3 * 16, "eight 16-byte stores a thread");
  {
    const int lv = lane & 31;
    const uint2 mine = digit_entry((uint32_t)(4 * wave + (lv & 3) + 32 * (lv >> 2)));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int src = (4 * i + (lane >> 4)) << 2;
      const uint32_t e0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mine.x);
      const uint32_t e1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mine.y);
      *reinterpret_cast<uint4 *>(tab + t * 16 + i * kThreads3 * 16) = make_uint4(e0, e1, e0, e1);
    }
  }
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

}  // namespace bqm
