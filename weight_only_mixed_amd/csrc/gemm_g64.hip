// Prefill and grouped dequant-GEMM instantiations: groups of 64 with byte or implied zero points.
#include "gemm_kernel.h"

namespace qp {
namespace gk {
QP_GEMM_VARIANT(64, kZpByte)
}  // namespace gk
}  // namespace qp
