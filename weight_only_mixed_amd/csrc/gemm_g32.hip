// Prefill and grouped dequant-GEMM instantiations: groups of 32 with byte or implied zero points.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_VARIANT(32, kZpByte)
}  // namespace gk
}  // namespace qp
