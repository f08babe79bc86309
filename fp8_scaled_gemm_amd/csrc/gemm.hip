// Scaled FP8 GEMM with per-tensor inverse scales: the instantiations of the
// kernels in gemm_kernels.hpp for alpha = fl32(inv_a * inv_b).
#include "gemm_kernels.hpp"

namespace fp8sg {

int device_cus() {
  constexpr int kMaxDevices = 64;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_gemm(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  return launch_gemm_any<false>(p, fa, fb, out, stream);
}

hipError_t launch_gemm_pair(const GemmProblem& p0, const GemmProblem& p1, int fa, int fb, int out,
                           hipStream_t stream) {
  // the backward pair: gradient codes (fa) x saved codes (fb)
  if (fa == FP8SG_E5M2 && fb == FP8SG_E4M3FN) {
    switch (out) {
      case FP8SG_OUT_BF16: return launch_tiles_pair<1, 0, FP8SG_OUT_BF16, false>(p0, p1, stream);
      case FP8SG_OUT_F16: return launch_tiles_pair<1, 0, FP8SG_OUT_F16, false>(p0, p1, stream);
      default: return launch_tiles_pair<1, 0, FP8SG_OUT_F32, false>(p0, p1, stream);
    }
  }
  hipError_t e = launch_gemm(p0, fa, fb, out, stream);
  if (e != hipSuccess) return e;
  return launch_gemm(p1, fa, fb, out, stream);
}

}  // namespace fp8sg
