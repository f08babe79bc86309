// The scaled GEMM with the GradScaler's unscale and non-finite check fused
// into the fp16 epilogue (used by the backward GEMMs, e5m2 gradient codes x
// e4m3 codes) [PT-CH20 §20.2.2: unscale the gradients, then check them for
// inf/NaN]: the kernels of gemm_kernels.hpp instantiated for the
// kOutF16Unscale output mode, with per-tensor or row-wise epilogue factors.  The
// stored values and the flag are those of an fp16 GEMM followed by the
// standalone unscale pass over its output.
#include "gemm_kernels.hpp"

namespace fp8sg {

hipError_t launch_gemm_unscale(const GemmProblem& p, int fa, int fb, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E4M3FN) return launch_tiles<0, 0, kOutF16Unscale, false>(p, stream);
  if (fa == FP8SG_E5M2 && fb == FP8SG_E4M3FN) return launch_tiles<1, 0, kOutF16Unscale, false>(p, stream);
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E5M2) return launch_tiles<0, 1, kOutF16Unscale, false>(p, stream);
  return launch_tiles<1, 1, kOutF16Unscale, false>(p, stream);
}

hipError_t launch_gemm_unscale_pair(const GemmProblem& p0, const GemmProblem& p1, bool rowwise,
                                    hipStream_t stream) {
  if (rowwise)  // epilogue factor fl32(inv_a[m] * inv_b[n]), then the unscale
    return launch_tiles_pair<FP8SG_E5M2, FP8SG_E4M3FN, kOutF16Unscale, true>(p0, p1, stream);
  return launch_tiles_pair<FP8SG_E5M2, FP8SG_E4M3FN, kOutF16Unscale, false>(p0, p1, stream);
}

}  // namespace fp8sg
