// Prefill dequant-GEMM instantiations: E4M3 scale bytes with a row factor and an fp16 fallback
// list (the layer GEMM; byte or implied zero points), every group size.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_VARIANT(128, kZpFp8)
QP_GEMM_VARIANT(64, kZpFp8)
QP_GEMM_VARIANT(32, kZpFp8)
}  // namespace gk
}  // namespace qp
