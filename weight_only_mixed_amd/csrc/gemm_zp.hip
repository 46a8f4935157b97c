// Prefill and grouped dequant-GEMM instantiations: zero points stored in b bits, every group size.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_VARIANT(128, kZpPacked)
QP_GEMM_VARIANT(64, kZpPacked)
QP_GEMM_VARIANT(32, kZpPacked)
}  // namespace gk
}  // namespace qp
