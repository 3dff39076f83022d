// Lloyd-Max codebook fit for the CQ codebooks cb2 / cb3 / cb4.
//
// "14MB holds 45M parameters: dissecting Needle's .cact file and W4A8
// quantization", section 1: the 4-, 8- and 16-level codebooks are fit offline
// by Lloyd-Max on 400,000 Gaussian samples for 200 iterations.
//
// The page gives no initialisation, symmetry rule or precision; this fit
// takes the reading (fp64 throughout, no FMA contraction in this file):
//   a_i = |z_i|; L/2 positive levels start at the interpolated order
//   statistics p_c = (c + 1/2)/(L/2): h = (n-1) p_c, j = floor(h),
//   level = a_(j) + (h - j) * (a_(j+1) - a_(j));
//   each iteration: boundaries at midpoints of adjacent levels (first cell
//   from 0, a sample on a boundary goes up); each level becomes its cell's
//   mean, the sum taken over blocks of 512 samples in index order and then
//   over the block sums in order; an empty cell keeps its level.
//   The L levels are the positive ones mirrored; the table is each level
//   rounded half-even to bfloat16 precision.
//
// One workgroup of 1024 threads.  Order statistics come from an 8-pass radix
// select over the bit patterns of |z| (non-negative doubles sort like their
// bit patterns).  In the iterations thread t owns sample block t.
#include "bqm_common.h"

namespace bqm {
namespace {

constexpr int kThreads = 1024;
constexpr int kSumBlock = 512;
constexpr int kMaxHalf = 8;

__device__ double radix_select(const double *z, int64_t n, int64_t k, unsigned *hist,
                               unsigned long long *sh_prefix, long long *sh_k) {
  const int t = threadIdx.x;
  unsigned long long prefix = 0, mask = 0;
  long long krem = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (t < 256) hist[t] = 0;
    __syncthreads();
    for (int64_t e = t; e < n; e += kThreads) {
      const unsigned long long key = (unsigned long long)__double_as_longlong(fabs(z[e]));
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255ull], 1u);
    }
    __syncthreads();
    if (t == 0) {
      long long cum = 0;
      int digit = 255;
      for (int d = 0; d < 256; ++d) {
        if (krem < cum + (long long)hist[d]) { digit = d; break; }
        cum += hist[d];
      }
      *sh_prefix = prefix | ((unsigned long long)digit << shift);
      *sh_k = krem - cum;
    }
    __syncthreads();
    prefix = *sh_prefix;
    krem = *sh_k;
    mask |= 255ull << shift;
    __syncthreads();
  }
  return __longlong_as_double((long long)prefix);
}

__global__ __launch_bounds__(kThreads) void codebook_fit_kernel(const double *__restrict__ z,
                                                                int64_t n, int levels, int iters,
                                                                double *__restrict__ raw,
                                                                float *__restrict__ table) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long sh_prefix;
  __shared__ long long sh_k;
  __shared__ double ostat[2 * kMaxHalf];
  __shared__ double pos[kMaxHalf];
  __shared__ double part[kThreads][kMaxHalf];
  __shared__ unsigned cpart[kThreads][kMaxHalf];
  const int t = threadIdx.x;
  const int half = levels / 2;
  const int nb = (int)((n + kSumBlock - 1) / kSumBlock);

  // ---- order statistics for the quantile start
  for (int c = 0; c < half; ++c) {
    const double p = ((double)c + 0.5) / (double)half;
    const double h = (double)(n - 1) * p;
    const int64_t j = (int64_t)floor(h);
    const int64_t j1 = (j + 1 < n) ? j + 1 : n - 1;
    const double lo = radix_select(z, n, j, hist, &sh_prefix, &sh_k);
    const double hi = radix_select(z, n, j1, hist, &sh_prefix, &sh_k);
    if (t == 0) {
      const double frac = h - (double)j;
      const double diff = hi - lo;
      const double step = frac * diff;
      pos[c] = lo + step;
      ostat[2 * c] = lo;
      ostat[2 * c + 1] = hi;
    }
    __syncthreads();
  }

  // ---- Lloyd iterations
  for (int it = 0; it < iters; ++it) {
    double bnd[kMaxHalf];
#pragma unroll
    for (int c = 0; c < kMaxHalf - 1; ++c)
      bnd[c] = (c < half - 1) ? 0.5 * (pos[c] + pos[c + 1]) : __builtin_inf();
    double acc[kMaxHalf];
    unsigned cnt[kMaxHalf];
#pragma unroll
    for (int c = 0; c < kMaxHalf; ++c) { acc[c] = 0.0; cnt[c] = 0; }
    if (t < nb) {
      const int64_t e0 = (int64_t)t * kSumBlock;
      const int64_t e1 = (e0 + kSumBlock < n) ? e0 + kSumBlock : n;
      for (int64_t e = e0; e < e1; ++e) {
        const double a = fabs(z[e]);
        int cell = 0;
#pragma unroll
        for (int c = 0; c < kMaxHalf - 1; ++c) cell += (bnd[c] <= a) ? 1 : 0;
#pragma unroll
        for (int c = 0; c < kMaxHalf; ++c) {
          const bool in = (cell == c);
          acc[c] = acc[c] + (in ? a : 0.0);
          cnt[c] += in ? 1u : 0u;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxHalf; ++c) { part[t][c] = acc[c]; cpart[t][c] = cnt[c]; }
    __syncthreads();
    if (t < half) {
      double s = 0.0;
      unsigned long long count = 0;
      for (int k = 0; k < nb; ++k) {
        s = s + part[k][t];
        count += cpart[k][t];
      }
      if (count > 0) pos[t] = s / (double)count;
    }
    __syncthreads();
  }

  if (t < half) {
    const double v = pos[t];
    const float bv = f64_to_bf16_rne(v);
    if (raw) {
      raw[half + t] = v;
      raw[half - 1 - t] = -v;
    }
    table[half + t] = bv;
    table[half - 1 - t] = -bv;
  }
}

}  // namespace

hipError_t launch_codebook_fit(const double *samples, int64_t n, int levels, int iters,
                               double *raw, float *table, hipStream_t s) {
  codebook_fit_kernel<<<1, kThreads, 0, s>>>(samples, n, levels, iters, raw, table);
  return hipGetLastError();
}

}  // namespace bqm
