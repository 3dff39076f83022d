// CQ GEMV kernels for 4-bit index fields, fp32 activations (A8 fused).
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(4, true, gemv_i4f)
}  // namespace bqm
