// Scaled FP8 GEMM with contraction-major operands (TA = true, TB = true; see
// k_gemm_pingpong): the instantiations for every format pair and output
// mode, the fused-unscale one included.  One file per operand mode so that
// the three compile in parallel.
#include "gemm_kernels.hpp"

namespace fp8sg {

hipError_t launch_gemm_km11(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (out != kOutF16Unscale) return launch_gemm_any<false, true, true>(p, fa, fb, out, stream);
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E4M3FN) return launch_tiles<0, 0, kOutF16Unscale, false, true, true>(p, stream);
  if (fa == FP8SG_E5M2 && fb == FP8SG_E4M3FN) return launch_tiles<1, 0, kOutF16Unscale, false, true, true>(p, stream);
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E5M2) return launch_tiles<0, 1, kOutF16Unscale, false, true, true>(p, stream);
  return launch_tiles<1, 1, kOutF16Unscale, false, true, true>(p, stream);
}

}  // namespace fp8sg
