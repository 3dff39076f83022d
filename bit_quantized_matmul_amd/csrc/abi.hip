// The C ABI of libbqm: argument checks, level tables, dispatch.
//
// Everything here runs on the host.  Arguments are validated before any HIP
// call, so a rejected call touches no device.  The only state kept is a
// per-device cache of (is gfx950, compute-unit count).
#include <math.h>
#include <string.h>

#include <mutex>

#include "bqm_common.h"

namespace bqm {

bool cq_gemv_supported(const bqm_cq_layout &L, bool fused);   // cq_gemv.hip

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxFitSamples = 1024 * 512;

struct DeviceInfo {
  bool probed = false;
  bool gfx950 = false;
  int num_cus = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Current device must be gfx950; returns its CU count, or a BQM error code.
int current_device(int *num_cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BQM_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return BQM_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo &d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BQM_EDEVICE;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.probed = true;
  }
  if (!d.gfx950) return BQM_ENOTSUP;
  *num_cus = d.num_cus;
  return BQM_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int index_bits_of(int bits) {
  switch (bits) {
    case BQM_CQ_BINARY: return 1;
    case BQM_CQ_B2: return 2;
    case BQM_CQ_B3: return 3;
    case BQM_CQ_B4: return 4;
    case BQM_CQ_TERNARY: return 2;
    default: return 0;                           // base-3 ternary too: not fixed-width fields
  }
}

int levels_of(int bits) {
  switch (bits) {
    case BQM_CQ_BINARY: return 2;
    case BQM_CQ_B2: return 4;
    case BQM_CQ_B3: return 8;
    case BQM_CQ_B4: return 16;
    case BQM_CQ_TERNARY:
    case BQM_CQ_TERNARY_B3: return 3;
    default: return 0;
  }
}

// Three-level Lloyd-Max optimum for N(0,1): c is the fixed point of
// c = E[Z | Z >= c/2] = phi(c/2) / Q(c/2), Q the upper tail.
double ternary_level() {
  double c = 1.0;
  for (int i = 0; i < 10000; ++i) {
    const double x = 0.5 * c;
    const double phi = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    const double tail = 0.5 * erfc(x / sqrt(2.0));
    const double nxt = phi / tail;
    if (nxt == c) break;
    c = nxt;
  }
  return c;
}

// Two-level optimum for N(0,1): E|Z| = sqrt(2/pi).
double binary_level() { return sqrt(2.0 / M_PI); }

uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

bool is_bf16_exact(float f) { return (__builtin_bit_cast(uint32_t, f) & 0xFFFFu) == 0; }

bool f16_exact(float f) { return (float)(_Float16)f == f; }

// 13 - max(floor(log2(max |level|)), -1) over the fp16 levels of the table
// (0 for an all-zero table): the GEMM scales a row's norms by 2^(this - E_M),
// E_M = floor(log2(the row's largest norm)), which keeps level x norm x scale
// and norm x scale below 2^15.
int fold_exp_of(const LevelTable &T) {
  float mx = 0.0f;
  for (int l = 0; l < T.levels; ++l) mx = fmaxf(mx, fabsf((float)__builtin_bit_cast(_Float16, T.h16[l])));
  int e = -1;
  if (mx > 0.0f) {
    int ex;
    frexpf(mx, &ex);                               // mx = f * 2^ex, f in [0.5, 1)
    e = ex - 1 > -1 ? ex - 1 : -1;
  }
  return 13 - e;
}

// Build the kernels' level table.  Fitted codebooks must be finite and
// bfloat16-representable (then they are exact in fp16 and bf16 alike).
int make_table(int bits, const float *codebook, LevelTable *T) {
  memset(T, 0, sizeof(*T));
  T->bits = bits;
  T->index_bits = index_bits_of(bits);
  T->levels = levels_of(bits);
  if (bits == BQM_CQ_BINARY || bits == BQM_CQ_TERNARY || bits == BQM_CQ_TERNARY_B3) {
    if (codebook != nullptr) return BQM_EINVAL;
    const double c = bits == BQM_CQ_BINARY ? binary_level() : ternary_level();
    const float cf = (float)c;
    const float sgn_bin[2] = {-1.0f, 1.0f};
    const float sgn_ter[3] = {-1.0f, 0.0f, 1.0f};
    const float *sg = bits == BQM_CQ_BINARY ? sgn_bin : sgn_ter;
    for (int l = 0; l < T->levels; ++l) {
      T->h16[l] = f32_to_f16_bits(sg[l]);
      T->b16[l] = (uint16_t)(__builtin_bit_cast(uint32_t, sg[l]) >> 16);
      T->f32[l] = sg[l] * cf;
    }
    T->cscale = cf;
    T->fold_exp = fold_exp_of(*T);
    return BQM_OK;
  }
  if (codebook == nullptr) return BQM_EINVAL;
  for (int l = 0; l < T->levels; ++l) {
    const float v = codebook[l];
    if (!isfinite(v) || !is_bf16_exact(v) || !f16_exact(v)) return BQM_EINVAL;
    T->h16[l] = f32_to_f16_bits(v);
    T->b16[l] = (uint16_t)(__builtin_bit_cast(uint32_t, v) >> 16);
    T->f32[l] = v;
  }
  T->cscale = 1.0f;
  T->fold_exp = fold_exp_of(*T);
  return BQM_OK;
}

int check_layout(const bqm_cq_layout *L) {
  if (!L) return BQM_EINVAL;
  bqm_cq_layout ref;
  if (cq_pack_info(L->rows, L->cols, L->group, L->bits, &ref) != BQM_OK) return BQM_EINVAL;
  if (memcmp(&ref, L, sizeof(ref)) != 0) return BQM_EINVAL;
  if (L->group != kGroup) return BQM_ENOTSUP;
  return BQM_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? BQM_OK : BQM_EDEVICE; }

constexpr int kGemvTokensForGemm = 32;   // cq_gemm: up to this many tokens run the batched GEMV kernel

// Scratch of cq_gemv_f32_noalloc: the int8 codes [batch, cols] and fp32
// scales [batch] that cq_gemv_f32 stages in q_out / scale_out, for up to
// kScratchBatch tokens of up to kScratchCols columns.  One copy per device
// (each device holds its own, until the process ends).  Host code never
// uses the array's name as an address: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr int kScratchBatch = 16;
constexpr int kScratchCols = 16384;
constexpr size_t kScratchCodes = (size_t)kScratchBatch * kScratchCols;   // 256 KiB of codes
constexpr size_t kScratchBytes = kScratchCodes + 256;                     // + the scales
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
uint8_t *g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(uint8_t **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BQM_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return BQM_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BQM_EDEVICE;
    g_scratch[dev] = static_cast<uint8_t *>(p);
  }
  *out = g_scratch[dev];
  return BQM_OK;
}

}  // namespace
}  // namespace bqm

using namespace bqm;

extern "C" {

int cq_pack_info(int rows, int cols, int group, int bits, bqm_cq_layout *layout) {
  if (!layout) return BQM_EINVAL;
  const int ib = index_bits_of(bits);
  const bool base3 = bits == BQM_CQ_TERNARY_B3;
  if (ib == 0 && !base3) return BQM_EINVAL;
  if (rows < 1 || cols < 1 || group < 2 || (group & (group - 1)) != 0) return BQM_EINVAL;
  if (cols % group != 0) return BQM_EINVAL;
  if (!base3 && ((int64_t)cols * ib) % 8 != 0) return BQM_EINVAL;
  bqm_cq_layout L;
  memset(&L, 0, sizeof(L));
  L.rows = rows;
  L.cols = cols;
  L.group = group;
  L.bits = bits;
  L.index_bits = ib;
  L.levels = levels_of(bits);
  // base-3: ceil(group / 5) bytes a group
  L.idx_row_bytes = base3 ? (int64_t)(cols / group) * ((group + 4) / 5) : (int64_t)cols * ib / 8;
  L.idx_bytes = (int64_t)rows * L.idx_row_bytes;
  L.norms_offset = (L.idx_bytes + 63) / 64 * 64;
  L.norms_count = (int64_t)rows * (cols / group);
  L.total_bytes = (L.norms_offset + 2 * L.norms_count + 63) / 64 * 64;
  *layout = L;
  return BQM_OK;
}

int cq_analytic_levels(int bits, float *levels) {
  if (!levels || (bits != BQM_CQ_BINARY && bits != BQM_CQ_TERNARY && bits != BQM_CQ_TERNARY_B3))
    return BQM_EINVAL;
  LevelTable T;
  make_table(bits, nullptr, &T);
  for (int l = 0; l < T.levels; ++l) levels[l] = T.f32[l];
  return BQM_OK;
}

int act_fwht_quant_a8(const float *x, int m, int k, int group, int8_t *q, float *scale,
                      bqm_stream_t stream) {
  if (!x || !q || !scale || m < 1 || k < 1 || group < 1 || (group & (group - 1))) return BQM_EINVAL;
  if (k % group) return BQM_EINVAL;
  if ((group != kGroup && group != 1) || k > 65536) return BQM_ENOTSUP;
  if (!aligned16(x) || !aligned16(q) || ((uintptr_t)scale & 3u)) return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  if (group == 1) return status_of(launch_act_quant_a8_unrotated(x, m, k, q, scale, (hipStream_t)stream));
  return status_of(launch_act_fwht_quant_a8(x, m, k, q, scale, (hipStream_t)stream));
}

int cq_gemv(const void *blob, const bqm_cq_layout *layout, const float *codebook, const int8_t *q,
            const float *scale, int batch, float *y, bqm_stream_t stream) {
  if (!blob || !q || !scale || !y || batch < 1) return BQM_EINVAL;
  int rc = check_layout(layout);
  if (rc) return rc;
  LevelTable T;
  rc = make_table(layout->bits, codebook, &T);
  if (rc) return rc;
  const bool base3 = layout->bits == BQM_CQ_TERNARY_B3;
  if (base3 ? !cq_gemv_t3_supported(*layout, batch) : (batch > 32 || !cq_gemv_supported(*layout, false)))
    return BQM_ENOTSUP;
  if (!aligned16(blob) || !aligned16(q) || ((uintptr_t)scale & 3u) || ((uintptr_t)y & 3u))
    return BQM_EALIGN;
  int cus;
  rc = current_device(&cus);
  if (rc) return rc;
  if (base3)
    return status_of(launch_cq_gemv_t3((const uint8_t *)blob, *layout, T, q, scale, batch, y, cus,
                                       (hipStream_t)stream));
  return status_of(launch_cq_gemv((const uint8_t *)blob, *layout, T, q, scale, batch, y, cus,
                                  (hipStream_t)stream));
}

int cq_gemv_f32(const void *blob, const bqm_cq_layout *layout, const float *codebook,
                const float *x, int batch, float *y, int8_t *q_out, float *scale_out,
                bqm_stream_t stream) {
  if (!blob || !x || !y || batch < 1) return BQM_EINVAL;
  int rc = check_layout(layout);
  if (rc) return rc;
  LevelTable T;
  rc = make_table(layout->bits, codebook, &T);
  if (rc) return rc;
  const bool base3 = layout->bits == BQM_CQ_TERNARY_B3;
  // rows too wide for the fused launch: the A8 step into the caller's code
  // buffers, then the cq_gemv product (as base-3 always does)
  const bool two_step = !base3 && !cq_gemv_supported(*layout, true) && q_out && scale_out &&
                        cq_gemv_supported(*layout, false);
  if (base3 ? (!cq_gemv_t3_supported(*layout, batch) || !q_out || !scale_out ||
               layout->cols > 65536)
            : (batch > 16 || !(two_step || cq_gemv_supported(*layout, true))))
    return BQM_ENOTSUP;
  if (!aligned16(blob) || !aligned16(x) || ((uintptr_t)q_out & 3u) || ((uintptr_t)scale_out & 3u) ||
      ((uintptr_t)y & 3u) || ((base3 || two_step) && !aligned16(q_out)))
    return BQM_EALIGN;
  int cus;
  rc = current_device(&cus);
  if (rc) return rc;
  if (two_step) {
    const hipError_t e = launch_act_fwht_quant_a8(x, batch, layout->cols, q_out, scale_out, (hipStream_t)stream);
    if (e != hipSuccess) return BQM_EDEVICE;
    return status_of(launch_cq_gemv((const uint8_t *)blob, *layout, T, q_out, scale_out, batch, y, cus,
                                    (hipStream_t)stream));
  }
  if (base3) {
    const hipError_t e = launch_act_fwht_quant_a8(x, batch, layout->cols, q_out, scale_out, (hipStream_t)stream);
    if (e != hipSuccess) return BQM_EDEVICE;
    return status_of(launch_cq_gemv_t3((const uint8_t *)blob, *layout, T, q_out, scale_out, batch, y, cus,
                                       (hipStream_t)stream));
  }
  return status_of(launch_cq_gemv_f32((const uint8_t *)blob, *layout, T, x, batch, y, q_out,
                                      scale_out, cus, (hipStream_t)stream));
}

int cq_gemv_lut(const void *blob, const bqm_cq_layout *layout, const int8_t *q, const float *scale, int batch,
                float *y, bqm_stream_t stream) {
  if (!blob || !q || !scale || !y || batch < 1) return BQM_EINVAL;
  int rc = check_layout(layout);
  if (rc) return rc;
  if (!cq_gemv_lut_supported(*layout, batch)) return BQM_ENOTSUP;
  LevelTable T;
  rc = make_table(layout->bits, nullptr, &T);
  if (rc) return rc;
  if (!aligned16(blob) || !aligned16(q) || ((uintptr_t)scale & 3u) || ((uintptr_t)y & 3u)) return BQM_EALIGN;
  int cus;
  rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_cq_gemv_lut((const uint8_t *)blob, *layout, T, q, scale, batch, y, cus,
                                      (hipStream_t)stream));
}

int cq_gemv_f32_noalloc(const void *blob, const bqm_cq_layout *layout, const float *codebook,
                        const float *x, int batch, float *y, bqm_stream_t stream) {
  if (!blob || !x || !y || batch < 1) return BQM_EINVAL;
  const int rc = check_layout(layout);
  if (rc) return rc;
  if (batch > kScratchBatch || layout->cols > kScratchCols) return BQM_ENOTSUP;   // past the scratch
  int cus;
  int rd = current_device(&cus);
  if (rd) return rd;
  uint8_t *sp = nullptr;
  rd = scratch_of_current_device(&sp);
  if (rd) return rd;
  // the codes at the start of the scratch, the scales 256-byte aligned after
  // the largest code block
  return cq_gemv_f32(blob, layout, codebook, x, batch, y, reinterpret_cast<int8_t *>(sp),
                     reinterpret_cast<float *>(sp + kScratchCodes), stream);
}

int cq_gemm(const void *blob, const bqm_cq_layout *layout, const float *codebook, const int8_t *q,
            const float *scale, int m, float *y, bqm_stream_t stream) {
  if (!blob || !q || !scale || !y || m < 1) return BQM_EINVAL;
  int rc = check_layout(layout);
  if (rc) return rc;
  LevelTable T;
  rc = make_table(layout->bits, codebook, &T);
  if (rc) return rc;
  // the kernel addresses the weights and activations with 32-bit offsets;
  // base-3 ternary: up to 16 tokens (and up to 16384 columns) run the batched
  // decode kernels, more on the base-3 GEMM
  const bool base3 = layout->bits == BQM_CQ_TERNARY_B3;
  const bool base3_small = base3 && m <= 16 && cq_t3_mma_supported(*layout, 2);
  if (layout->idx_bytes >= (int64_t)1 << 30 || (int64_t)m * layout->cols >= (int64_t)1 << 30 ||
      (base3 && !base3_small && !cq_t3_gemm_supported(*layout, m)))
    return BQM_ENOTSUP;
  if (!aligned16(blob) || !aligned16(q) || ((uintptr_t)scale & 3u) || ((uintptr_t)y & 3u))
    return BQM_EALIGN;
  int cus;
  rc = current_device(&cus);
  if (rc) return rc;
  if (base3_small)
    return status_of(m >= 2 ? launch_cq_t3_mma((const uint8_t *)blob, *layout, T, q, scale, m, y, cus,
                                               (hipStream_t)stream)
                            : launch_cq_gemv_t3((const uint8_t *)blob, *layout, T, q, scale, 1, y, cus,
                                                (hipStream_t)stream));
  if (base3)
    return status_of(launch_cq_t3_gemm((const uint8_t *)blob, *layout, T, q, scale, m, y, cus,
                                       (hipStream_t)stream));
  // up to 32 tokens: the batched decode kernel reads the weights once for all
  // of them and beats the GEMM's few tiles (measured at 32 tokens: 4096x4096
  // 8.5 against 19.0 us, 14336x4096 15.2 against 24.1, 4096x14336 21.8
  // against 54.8; at 64 tokens, in two launches, the GEMM wins on three of
  // the four shapes)
  // Up to 64 tokens, where even 64 x 64 GEMM tiles would leave CUs idle, the
  // same in launches of 32 (at 64 tokens: 4096x4096 17.0 against 19.2 us,
  // 4096x14336 43.6 against 54.4; 14336x4096 fills the CUs with 64 x 64 tiles
  // and keeps the GEMM, 24.8 against 30.4)
  const int64_t t64 = (int64_t)((m + 63) / 64) * ((layout->rows + 63) / 64);
  const bool few = m <= kGemvTokensForGemm || (m <= 2 * kGemvTokensForGemm && t64 < (int64_t)cus * 7 / 8);
  if (few && cq_gemv_mma_supported(*layout, 16)) {
    for (int b0 = 0; b0 < m; b0 += kGemvTokensForGemm) {
      const int nb = m - b0 < kGemvTokensForGemm ? m - b0 : kGemvTokensForGemm;
      const hipError_t e = launch_cq_gemv((const uint8_t *)blob, *layout, T, q + (size_t)b0 * layout->cols,
                                          scale + b0, nb, y + (size_t)b0 * layout->rows, cus, (hipStream_t)stream);
      if (e != hipSuccess) return BQM_EDEVICE;
    }
    return BQM_OK;
  }
  return status_of(launch_cq_gemm((const uint8_t *)blob, *layout, T, q, scale, m, y, cus,
                                  (hipStream_t)stream));
}

int q4_0_gemv(const void *blocks, int rows, int cols, const float *x, int batch, float *y,
              bqm_stream_t stream) {
  if (!blocks || !x || !y || rows < 1 || cols < 1 || batch < 1) return BQM_EINVAL;
  // the kernel addresses the blocks with 32-bit offsets
  if (batch > 16 || (int64_t)rows * (((int64_t)cols + 31) / 32) * 18 >= ((int64_t)1 << 31))
    return BQM_ENOTSUP;
  if (!aligned16(blocks) || !aligned16(x) || ((uintptr_t)y & 3u)) return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(
      launch_q4_0_gemv((const uint8_t *)blocks, rows, cols, x, batch, y, cus, (hipStream_t)stream));
}

int q4_0_gemm(const void *blocks, int rows, int cols, const float *x, int m, float *y,
              bqm_stream_t stream) {
  if (!blocks || !x || !y || rows < 1 || cols < 1 || m < 1) return BQM_EINVAL;
  if (!aligned16(blocks) || !aligned16(x) || ((uintptr_t)y & 3u)) return BQM_EALIGN;
  const int64_t nblk = ((int64_t)cols + 31) / 32;
  if ((int64_t)rows * nblk * 18 >= ((int64_t)1 << 31) || (int64_t)m * cols * 4 >= ((int64_t)1 << 31) ||
      ((int64_t)m + 63) / 64 > 65535)
    return BQM_ENOTSUP;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_q4_0_gemm((const uint8_t *)blocks, rows, cols, x, m, y, cus, (hipStream_t)stream));
}

int q4_0_gemv_a8(const void *blocks, int rows, int cols, const int8_t *q, const float *scale, int batch,
                 float *y, bqm_stream_t stream) {
  if (!blocks || !q || !scale || !y || rows < 1 || cols < 1 || batch < 1) return BQM_EINVAL;
  // 32-bit offsets for the blocks and the codes
  if (batch > 16 || (int64_t)rows * (((int64_t)cols + 31) / 32) * 18 >= ((int64_t)1 << 31) ||
      (int64_t)batch * cols >= ((int64_t)1 << 31))
    return BQM_ENOTSUP;
  if (!aligned16(blocks) || !aligned16(q) || ((uintptr_t)scale & 3u) || ((uintptr_t)y & 3u)) return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_q4_0_gemv_a8((const uint8_t *)blocks, rows, cols, q, scale, batch, y, (hipStream_t)stream));
}

int q4_0_gemv_a8_f32(const void *blocks, int rows, int cols, const float *x, int batch, float *y,
                     int8_t *q_out, float *scale_out, bqm_stream_t stream) {
  if (!blocks || !x || !y || rows < 1 || cols < 1 || batch < 1) return BQM_EINVAL;
  // 32-bit offsets for the blocks; one token's codes must fit a workgroup's LDS
  if (batch > 16 || (int64_t)rows * (((int64_t)cols + 31) / 32) * 18 >= ((int64_t)1 << 31) ||
      !q4_0_gemv_a8_fused_supported(cols, batch))
    return BQM_ENOTSUP;
  if (!aligned16(blocks) || ((uintptr_t)x & 3u) || ((uintptr_t)y & 3u) || ((uintptr_t)scale_out & 3u))
    return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_q4_0_gemv_a8_fused((const uint8_t *)blocks, rows, cols, x, batch, y, q_out, scale_out,
                                             cus, (hipStream_t)stream));
}

int q4_0_gemm_a8(const void *blocks, int rows, int cols, const int8_t *q, const float *scale, int m, float *y,
                 bqm_stream_t stream) {
  if (!blocks || !q || !scale || !y || rows < 1 || cols < 1 || m < 1) return BQM_EINVAL;
  if ((int64_t)rows * (((int64_t)cols + 31) / 32) * 18 >= ((int64_t)1 << 31) ||
      (int64_t)m * cols >= ((int64_t)1 << 31) || ((int64_t)m + 31) / 32 > 65535)
    return BQM_ENOTSUP;
  if (!aligned16(blocks) || !aligned16(q) || ((uintptr_t)scale & 3u) || ((uintptr_t)y & 3u)) return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_q4_0_gemm_a8((const uint8_t *)blocks, rows, cols, q, scale, m, y, cus,
                                       (hipStream_t)stream));
}

int cq_pack(const float *w, const bqm_cq_layout *layout, const float *codebook, void *blob,
            int32_t *status, bqm_stream_t stream) {
  if (!w || !blob) return BQM_EINVAL;
  int rc = check_layout(layout);
  if (rc) return rc;
  LevelTable T;
  rc = make_table(layout->bits, codebook, &T);
  if (rc) return rc;
  if (!aligned16(w) || !aligned16(blob) || ((uintptr_t)status & 3u)) return BQM_EALIGN;
  int cus;
  rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_cq_pack(w, *layout, T, (uint8_t *)blob, status, (hipStream_t)stream));
}

int q4_0_pack(const float *w, int rows, int cols, void *blocks, bqm_stream_t stream) {
  if (!w || !blocks || rows < 1 || cols < 1) return BQM_EINVAL;
  if (!aligned16(w) || !aligned16(blocks)) return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_q4_0_pack(w, rows, cols, (uint8_t *)blocks, (hipStream_t)stream));
}

int cq_codebook_fit(const double *samples, int64_t n, int levels, int iters, double *raw,
                    float *table, bqm_stream_t stream) {
  if (!samples || !table || n < 2 || iters < 0) return BQM_EINVAL;
  if (levels != 2 && levels != 4 && levels != 8 && levels != 16) return BQM_EINVAL;
  if (n > kMaxFitSamples) return BQM_ENOTSUP;
  if (((uintptr_t)samples & 7u) || ((uintptr_t)raw & 7u) || ((uintptr_t)table & 3u))
    return BQM_EALIGN;
  int cus;
  const int rc = current_device(&cus);
  if (rc) return rc;
  return status_of(launch_codebook_fit(samples, n, levels, iters, raw, table, (hipStream_t)stream));
}

const char *bqm_strerror(int code) {
  switch (code) {
    case BQM_OK: return "ok";
    case BQM_EINVAL: return "invalid argument";
    case BQM_EALIGN: return "misaligned pointer";
    case BQM_ENOTSUP: return "not supported";
    case BQM_EDEVICE: return "device error";
    case BQM_ERANGE: return "value out of range";
    default: return "unknown error";
  }
}

}  // extern "C"
