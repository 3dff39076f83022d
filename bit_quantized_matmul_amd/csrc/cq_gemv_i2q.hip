// CQ GEMV kernels for 2-bit index fields, int8 activations.
#include "cq_gemv_impl.h"

namespace bqm {
BQM_GEMV_VARIANT(2, false, gemv_i2q)
}  // namespace bqm
