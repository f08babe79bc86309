// Small linear layers in one launch per pass [FP8-TRAIN §2 (amax, fp64 scale,
// cast), §4 (the forward, dgrad and wgrad products)].  At sizes such as
// B = 64, K = 128, N = 256 every kernel is mostly launch and dependency
// latency, so the number of launches sets the time.
//
// Forward: every block of the forward GEMM reduces |x| and |W| over the whole
// tensors itself (at most 64 Ki elements each, read from L2), derives both
// scales, casts the rows of x and W its tile needs on their way into LDS and
// multiplies them; the blocks in the first tile column store x's codes, those
// in the first tile row W's codes, and block (0, 0) the two records.  One
// launch instead of a cast launch and a GEMM launch.
//
// Backward: dgrad and wgrad tiles share one launch (blockIdx.z picks the
// problem); every block reduces |gy| and casts the parts of gy its tile needs
// (rows for dgrad, columns for wgrad), the saved codes of W and x are read
// contraction-major; the dgrad blocks of the first tile column store gy's
// codes and block (0, 0, 0) its record.  One launch instead of two.
//
// The codes, records and outputs are those of the cast kernels followed by
// the GEMM kernels, bit for bit: the same quantization (quant8 at scale32),
// the same fp64 scale and inverse, the same MFMA k order, the same epilogue.
// No transposed copies are made (the backward reads the codes
// contraction-major).
#include "gemm_kernels.hpp"

namespace fp8sg {

constexpr int kSmallThreads = 256;
using SmallCfg = GemmCfg<128, 128, 2, 2>;
static_assert(SmallCfg::kThreads == kSmallThreads, "one block shape");

// max |x| over n bf16 values (n a multiple of 8), every thread of the block
// gets it; canonical NaN for any NaN.  The partial maxima meet in the
// kernel's dynamic LDS, before the GEMM uses it.
__device__ __forceinline__ uint32_t block_absmax_bits(const uint16_t* x, int64_t n, uint32_t* red) {
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nv = n >> 3;
  uint32_t m = 0;
  constexpr int kU = 8;  // loads in flight per thread; past the end a lane rereads vector 0
  for (int64_t k0 = threadIdx.x; k0 < nv; k0 += (int64_t)kSmallThreads * kU) {
    uint4 t[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + (int64_t)u * kSmallThreads;
      t[u] = xv[k < nv ? k : 0];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) m = absmax8(m, t[u]);
  }
  uint32_t b = wave_max_u32(absmax_bits(m));
  __syncthreads();  // red may hold an earlier reduction's values
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = b;
  __syncthreads();
  b = red[0];
#pragma unroll
  for (int w = 1; w < kSmallThreads / kWave; ++w) b = red[w] > b ? red[w] : b;
  return b;
}

// A record as the one-block cast leaves it: its amax as the single partial
// maximum, then amax and the scale fields.
__device__ __forceinline__ void write_self_record(fp8sg_scale_rec* rec, uint32_t bits,
                                                  const ScaleVals& v) {
  rec->_part[0] = bits;
  rec->_nparts = 1;
  rec->amax = __uint_as_float(bits);
  rec->scale = v.s;
  rec->inv = v.inv;
  rec->scale32 = v.s32;
  rec->inv32 = v.inv32;
}

template <int OUT>
__global__ __launch_bounds__(kSmallThreads) void k_small_fwd(SmallFwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t* red = reinterpret_cast<uint32_t*>(smem);
  const uint32_t bx_bits = block_absmax_bits(a.x, a.p.M * a.p.K, red);
  const uint32_t bw_bits = block_absmax_bits(a.w, a.p.N * a.p.K, red);
  __syncthreads();  // the GEMM's tiles overwrite red
  const ScaleVals sx = scale_from_amax(__uint_as_float(bx_bits), FP8SG_E4M3FN);
  const ScaleVals sw = scale_from_amax(__uint_as_float(bw_bits), FP8SG_E4M3FN);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    write_self_record(a.x_sc, bx_bits, sx);
    write_self_record(a.w_sc, bw_bits, sw);
  }
  const CastSrc cx{a.x, sx.s32, sx.inv, blockIdx.x == 0 ? a.x_q : nullptr};
  const CastSrc cw{a.w, sw.s32, sw.inv, blockIdx.y == 0 ? a.w_q : nullptr};
  gemm_small_tile<128, 128, 2, 2, FP8SG_E4M3FN, FP8SG_E4M3FN, OUT, false, false, false, true, true>(
      a.p, blockIdx.x, blockIdx.y, cx, cw);
}

template <int OUT>
__global__ __launch_bounds__(kSmallThreads) void k_small_bwd(SmallBwdArgs a) {
  const int64_t pm = blockIdx.z ? a.wg.M : a.dg.M, pn = blockIdx.z ? a.wg.N : a.dg.N;
  if ((int64_t)blockIdx.y * 128 >= pm || (int64_t)blockIdx.x * 128 >= pn) return;  // whole block
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t* red = reinterpret_cast<uint32_t*>(smem);
  const uint32_t bg_bits = block_absmax_bits(a.gy, a.rows * a.cols, red);
  __syncthreads();  // the GEMM's tiles overwrite red
  const ScaleVals sg = scale_from_amax(__uint_as_float(bg_bits), FP8SG_E5M2);
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
    write_self_record(a.gy_sc, bg_bits, sg);
  // gy's codes are stored by the dgrad blocks of the first tile column
  const CastSrc cg{a.gy, sg.s32, sg.inv, blockIdx.z == 0 && blockIdx.x == 0 ? a.gy_q : nullptr};
  if (blockIdx.z == 0)  // dgrad: gy rows cast, W codes as B^T
    gemm_small_tile<128, 128, 2, 2, FP8SG_E5M2, FP8SG_E4M3FN, OUT, false, false, true, true, false>(
        a.dg, blockIdx.x, blockIdx.y, cg);
  else  // wgrad: gy as A^T cast, x codes as B^T
    gemm_small_tile<128, 128, 2, 2, FP8SG_E5M2, FP8SG_E4M3FN, OUT, false, true, true, true, false>(
        a.wg, blockIdx.x, blockIdx.y, cg);
}

bool small_layer_fits(int64_t M, int64_t N, int64_t K) {
  return M * K <= kSelfCastMaxElems && N * K <= kSelfCastMaxElems && M * N <= kSelfCastMaxElems;
}

hipError_t launch_small_fwd(const SmallFwdArgs& a, int out, hipStream_t stream) {
  const dim3 grid((unsigned)((a.p.N + 127) / 128), (unsigned)((a.p.M + 127) / 128));
  const size_t lds = SmallCfg::kLdsBytes;
  switch (out) {
    case FP8SG_OUT_BF16: hipLaunchKernelGGL(k_small_fwd<FP8SG_OUT_BF16>, grid, dim3(kSmallThreads), lds, stream, a); break;
    case FP8SG_OUT_F16: hipLaunchKernelGGL(k_small_fwd<FP8SG_OUT_F16>, grid, dim3(kSmallThreads), lds, stream, a); break;
    default: hipLaunchKernelGGL(k_small_fwd<FP8SG_OUT_F32>, grid, dim3(kSmallThreads), lds, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_small_bwd(const SmallBwdArgs& a, int out, hipStream_t stream) {
  auto cdiv = [](int64_t x, int64_t y) { return (x + y - 1) / y; };
  const int64_t gx = cdiv(a.dg.N, 128) > cdiv(a.wg.N, 128) ? cdiv(a.dg.N, 128) : cdiv(a.wg.N, 128);
  const int64_t gy = cdiv(a.dg.M, 128) > cdiv(a.wg.M, 128) ? cdiv(a.dg.M, 128) : cdiv(a.wg.M, 128);
  const dim3 grid((unsigned)gx, (unsigned)gy, 2);
  const size_t lds = SmallCfg::kLdsBytes;
  switch (out) {
    case FP8SG_OUT_BF16: hipLaunchKernelGGL(k_small_bwd<FP8SG_OUT_BF16>, grid, dim3(kSmallThreads), lds, stream, a); break;
    case FP8SG_OUT_F16: hipLaunchKernelGGL(k_small_bwd<FP8SG_OUT_F16>, grid, dim3(kSmallThreads), lds, stream, a); break;
    case kOutF16Unscale: hipLaunchKernelGGL(k_small_bwd<kOutF16Unscale>, grid, dim3(kSmallThreads), lds, stream, a); break;
    default: hipLaunchKernelGGL(k_small_bwd<FP8SG_OUT_F32>, grid, dim3(kSmallThreads), lds, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace fp8sg
