// CQ GEMV kernels for 4-bit index fields, int8 activations.
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(4, false, gemv_i4q)
}  // namespace bqm
