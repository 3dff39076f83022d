// CQ GEMV kernels for 1-bit index fields, fp32 activations (A8 fused).
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(1, true, gemv_i1f)
}  // namespace bqm
