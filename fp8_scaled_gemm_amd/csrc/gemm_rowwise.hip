// Scaled FP8 GEMM with row-wise inverse-scale vectors: the instantiations of
// the kernels in gemm_kernels.hpp whose epilogue multiplies element (m, n) by
// fl32(inv_a[m] * inv_b[n]) [FP8-TRAIN §1].  A separate translation unit, so
// the two sets of kernels compile in parallel.
#include "gemm_kernels.hpp"

namespace fp8sg {

hipError_t launch_gemm_rowwise(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  return launch_gemm_any<true>(p, fa, fb, out, stream);
}

// The row-wise backward pair (e5m2 gradient codes x e4m3 codes): one launch
// of the 128 x 128 kernel when both are small, otherwise one launch each.
hipError_t launch_gemm_rowwise_pair(const GemmProblem& p0, const GemmProblem& p1, int out,
                                    hipStream_t stream) {
  switch (out) {
    case FP8SG_OUT_BF16: return launch_tiles_pair<1, 0, FP8SG_OUT_BF16, true>(p0, p1, stream);
    case FP8SG_OUT_F16: return launch_tiles_pair<1, 0, FP8SG_OUT_F16, true>(p0, p1, stream);
    default: return launch_tiles_pair<1, 0, FP8SG_OUT_F32, true>(p0, p1, stream);
  }
}

}  // namespace fp8sg
