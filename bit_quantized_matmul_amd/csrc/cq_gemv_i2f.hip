// CQ GEMV kernels for 2-bit index fields, fp32 activations (A8 fused).
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(2, true, gemv_i2f)
}  // namespace bqm
