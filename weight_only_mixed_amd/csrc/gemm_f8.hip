// Prefill dequant-GEMM instantiations: E4M3 scale bytes with a row factor and an fp16 fallback
// list (byte or implied zero points), the layer GEMM at every group size; the grouped halves
// are in gemm_f8_grouped_g*.hip.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_LAYER(128, kZpFp8)
QP_GEMM_LAYER(64, kZpFp8)
QP_GEMM_LAYER(32, kZpFp8)
}  // namespace gk
}  // namespace qp
