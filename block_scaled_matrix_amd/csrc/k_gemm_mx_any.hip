// k_gemm_mx_any.hip - launches of the general block-scaled kernel (gemm_mx_any.hpp) for
// K-major operands: every pairing of E4M3, E5M2, E2M3, E3M2, E2M1 except the ones the
// tuned kernel of k_gemm_mx.hip runs.
#include "gemm_mx_any.hpp"

namespace bsm {

hipError_t launch_gemm_mx_any(const GemmArgs& a, hipStream_t st) { return mxany::launch_formats<false, false>(a, st); }

}  // namespace bsm
