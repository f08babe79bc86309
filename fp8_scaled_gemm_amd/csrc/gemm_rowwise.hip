// Scaled FP8 GEMM with row-wise inverse-scale vectors: the instantiations of
// the kernels in gemm_kernels.hpp whose epilogue multiplies element (m, n) by
// fl32(inv_a[m] * inv_b[n]) [FP8-TRAIN §1].  A separate translation unit, so
// the two sets of kernels compile in parallel.
#include "gemm_kernels.hpp"

namespace fp8sg {

hipError_t launch_gemm_rowwise(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  return launch_gemm_any<true>(p, fa, fb, out, stream);
}

}  // namespace fp8sg
