// Scaled FP8 GEMM with per-tensor inverse scales: the instantiations of the
// kernels in gemm_kernels.hpp for alpha = fl32(inv_a * inv_b).
#include "gemm_kernels.hpp"

namespace fp8sg {

hipError_t launch_gemm(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  return launch_gemm_any<false>(p, fa, fb, out, stream);
}

}  // namespace fp8sg
