// CQ GEMV kernels for 3-bit index fields, fp32 activations (A8 fused).
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(3, true, gemv_i3f)
}  // namespace bqm
