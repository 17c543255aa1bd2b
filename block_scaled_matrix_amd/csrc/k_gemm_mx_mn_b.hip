// k_gemm_mx_mn_b.hip - launches of the general block-scaled kernel (gemm_mx_any.hpp) with
// A K-major, B MN-major (an MN-major operand: K rows, M or N contiguous; E4M3, E5M2 or E2M1).
// One translation unit per major-order combination, so the instances compile in parallel.
#include "gemm_mx_any.hpp"

namespace bsm {

hipError_t launch_gemm_mx_mn_b(const GemmArgs& a, hipStream_t st) { return mxany::launch_formats<false, true>(a, st); }

}  // namespace bsm
