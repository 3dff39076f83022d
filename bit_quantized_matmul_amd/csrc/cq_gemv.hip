// Decode GEMV on packed CQ weights: entry points.  The kernel and its host
// dispatch are in cq_gemv_impl.h; each (index bits, fused) set of kernels is
// compiled in its own cq_gemv_i<IB><f|q>.hip.
#include "cq_gemv_impl.h"

namespace bqm {

#define BQM_GEMV_DECL(NAME)                                                                   \
  hipError_t NAME(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,          \
                  const int8_t *q, const float *scale, const float *x, int8_t *q_out,         \
                  float *scale_out, int batch, float *y, int num_cus, hipStream_t s);
BQM_GEMV_DECL(gemv_i1q)
BQM_GEMV_DECL(gemv_i1f)
BQM_GEMV_DECL(gemv_i2q)
BQM_GEMV_DECL(gemv_i2f)
BQM_GEMV_DECL(gemv_i3q)
BQM_GEMV_DECL(gemv_i3f)
BQM_GEMV_DECL(gemv_i4q)
BQM_GEMV_DECL(gemv_i4f)

bool cq_gemv_supported(const bqm_cq_layout &L, bool fused) {
  GemvConfig cfg;
  if (L.cols % kGroup) return false;
  if ((size_t)L.cols * 2 > kMaxActLds) return false;       // one token's fp16 copy must fit
  if (fused && L.cols > kMaxFusedCols) return false;
  if ((uint64_t)L.idx_bytes >= kIdxLimit || (uint64_t)L.norms_count * 2 >= kIdxLimit) return false;
  return choose_config(1 << 20, L.cols / kChunk, 1, 256, cfg);
}

hipError_t launch_cq_gemv(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                          const int8_t *q, const float *scale, int batch, float *y,
                          int num_cus, hipStream_t s) {
  // From 2 tokens on (3 for rows past 4096 columns), one pass over the
  // weights on the matrix cores serves them all (the VALU GEMV re-reads every
  // weight per launch of 4 tokens and spends its time on the dot products);
  // past 4 tokens, rows the batched GEMV does not take go to the GEMM kernel.
  if (cq_gemv_mma_supported(L, batch))
    return launch_cq_gemv_mma(blob, L, T, q, scale, batch, y, num_cus, s);
  if (batch > 4 && L.idx_bytes < ((int64_t)1 << 30))
    return launch_cq_gemm(blob, L, T, q, scale, batch, y, num_cus, s);
  switch (L.index_bits) {
    case 1: return gemv_i1q(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
    case 2: return gemv_i2q(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
    case 3: return gemv_i3q(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
    default: return gemv_i4q(blob, L, T, q, scale, nullptr, nullptr, nullptr, batch, y, num_cus, s);
  }
}

hipError_t launch_cq_gemv_f32(const uint8_t *blob, const bqm_cq_layout &L, const LevelTable &T,
                              const float *x, int batch, float *y, int8_t *q_out,
                              float *scale_out, int num_cus, hipStream_t s) {
  const bool matrix_cores = cq_gemv_mma_supported(L, batch) ||
                            (batch > 4 && L.idx_bytes < ((int64_t)1 << 30));
  if (matrix_cores && q_out && scale_out && ((uintptr_t)q_out & 15u) == 0) {
    // the A8 step into the caller's code and scale buffers, then the same
    // matrix-core product as launch_cq_gemv
    const hipError_t e = launch_act_fwht_quant_a8(x, batch, L.cols, q_out, scale_out, s);
    if (e != hipSuccess) return e;
    return launch_cq_gemv(blob, L, T, q_out, scale_out, batch, y, num_cus, s);
  }
  switch (L.index_bits) {
    case 1: return gemv_i1f(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
    case 2: return gemv_i2f(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
    case 3: return gemv_i3f(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
    default: return gemv_i4f(blob, L, T, nullptr, nullptr, x, q_out, scale_out, batch, y, num_cus, s);
  }
}

}  // namespace bqm
