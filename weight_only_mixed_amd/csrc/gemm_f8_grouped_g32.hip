// Grouped (routed-expert) dequant-GEMM instantiations: E4M3 scale bytes with a row factor and
// an fp16 fallback list per expert, groups of 32.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_GROUPED(32, kZpFp8)
}  // namespace gk
}  // namespace qp
