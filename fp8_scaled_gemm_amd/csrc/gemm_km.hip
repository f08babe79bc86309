// Scaled FP8 GEMM with contraction-major operands: dispatch over the operand
// modes (gemm_km01/10/11.hip hold the instantiations), and the backward pair
// of a linear layer without transposed copies [FP8-TRAIN §4 backward]:
//   dgrad gx = gy W:   A = gy codes [M, N] (row-major), B = W codes [N, K]
//                      (contraction-major: TB);
//   wgrad gW = gy^T x: A = gy codes [M, N], B = x codes [M, K] (both
//                      contraction-major: TA, TB).
// The products and their k order are those of the GEMMs on transposed copies,
// so the outputs are the same bits.
#include "gemm_kernels.hpp"

namespace fp8sg {

hipError_t launch_gemm_km01(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream);
hipError_t launch_gemm_km10(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream);
hipError_t launch_gemm_km11(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream);

void linear_copies(int64_t M, int64_t N, int64_t K, bool& x_t, bool& w_t, bool& gy_t) {
  // dgrad (M x K over N) reads W in the B slot: a contraction-major read
  // costs nothing there.  wgrad (N x K over M): the operand in the A slot
  // keeps its copy -- x where the launcher swaps the roles, else gy -- when
  // it takes the large-tile kernel (read contraction-major there it makes
  // that GEMM about 5% slower); small layers keep none (both backward GEMMs
  // then share one launch of the 128 x 128 kernel, or each pass is one
  // launch).  The choice is the GEMMs' alone: the copy costs its cast one
  // more byte per element, which at the MLP block's shapes about cancels
  // what the GEMM saves.
  w_t = false;
  x_t = gy_t = false;
  if (!big_tiles_wanted(N, K)) return;
  if (big_tiling(N, K, device_cus(), true) == kTile224Swapped) x_t = true;
  else gy_t = true;
}

hipError_t launch_gemm_km(const GemmProblem& p, int fa, int fb, int out, bool ta, bool tb,
                          hipStream_t stream) {
  if (ta && tb) return launch_gemm_km11(p, fa, fb, out, stream);
  if (ta) return launch_gemm_km10(p, fa, fb, out, stream);
  if (tb) return launch_gemm_km01(p, fa, fb, out, stream);
  return out == kOutF16Unscale ? launch_gemm_unscale(p, fa, fb, stream) : launch_gemm(p, fa, fb, out, stream);
}

template <int OUT>
static hipError_t launch_pair_small(const GemmProblem& dg, const GemmProblem& wg, hipStream_t stream) {
  // e5m2 gradient codes x e4m3 codes; dgrad (row-major A, contraction-major B)
  // and wgrad (both contraction-major) in one launch of the 128 x 128 kernel
  return launch_tiles_pair<1, 0, OUT, false, false, true, true, true>(dg, wg, stream);
}

hipError_t launch_gemm_km_pair(const GemmProblem& dg, const GemmProblem& wg, int out, hipStream_t stream) {
  auto big = [](const GemmProblem& p, bool ta) {
    return ((p.M + 255) / 256) * ((p.N + 255) / 256) >= 128 &&
           (ta ? big_tiles_fit<true, true>(p) : big_tiles_fit<false, true>(p));
  };
  if (big(dg, false) || big(wg, true)) {
    hipError_t e = launch_gemm_km01(dg, FP8SG_E5M2, FP8SG_E4M3FN, out, stream);
    if (e != hipSuccess) return e;
    return launch_gemm_km11(wg, FP8SG_E5M2, FP8SG_E4M3FN, out, stream);
  }
  switch (out) {
    case FP8SG_OUT_BF16: return launch_pair_small<FP8SG_OUT_BF16>(dg, wg, stream);
    case FP8SG_OUT_F16: return launch_pair_small<FP8SG_OUT_F16>(dg, wg, stream);
    case kOutF16Unscale: return launch_pair_small<kOutF16Unscale>(dg, wg, stream);
    default: return launch_pair_small<FP8SG_OUT_F32>(dg, wg, stream);
  }
}

}  // namespace fp8sg
