// CQ GEMV kernels for 1-bit index fields, int8 activations.
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(1, false, gemv_i1q)
}  // namespace bqm
