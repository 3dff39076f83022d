// CQ GEMV kernels for 3-bit index fields, int8 activations.
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(3, false, gemv_i3q)
}  // namespace bqm
