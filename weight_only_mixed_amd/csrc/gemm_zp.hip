// Prefill and grouped dequant-GEMM instantiations: zero points stored in b bits, every group size.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_VARIANT(128, true)
QP_GEMM_VARIANT(64, true)
QP_GEMM_VARIANT(32, true)
}  // namespace gk
}  // namespace qp
