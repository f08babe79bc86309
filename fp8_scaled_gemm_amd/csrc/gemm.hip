// Scaled FP8 GEMM on gfx950 matrix cores:
//   C[M,N] = out( (sum_k dec(A[m,k]) * dec(B[n,k])) * fl32(inv_a * inv_b) )
// [FP8-TRAIN §2 (dequantise by the product of the two inverse scales), §4 (the
// forward, dgrad and wgrad products), AMP-MP "不要忘记 Accumulator Precision"
// (low-precision multiply, fp32 accumulate)].
//
// Both operands are contiguous along the contraction (the quantizer writes the
// transposed copies the backward GEMMs need), so one kernel form serves all
// three GEMMs.  Every FP8 x FP8 product is exact in fp32 and the matrix cores
// accumulate in fp32; only the summation order differs from a sequential loop.
//
// Structure: a BM x BN block tile per workgroup, K consumed 128 bytes at a
// time.  Each k-tile of A and B is fetched with 16-byte global loads into
// registers while the previous tile is being multiplied, then written to the
// other half of a double-buffered LDS tile (16-byte chunks XOR-swizzled by row
// so the fragment reads hit distinct banks).  Each wave owns a (BM/WM) x
// (BN/WN) sub-tile made of 16x16 blocks and issues
// v_mfma_f32_16x16x128_f8f6f4 with the operand formats (e4m3 = 0, e5m2 = 1)
// selected per operand.  The B fragment is passed as the instruction's first
// source so each lane's four accumulators are four consecutive output
// columns, stored as one 8-byte (bf16/fp16) or 16-byte (fp32) write.
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;  // bytes (= FP8 elements) of K per tile

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kTM = BM / WM / 16;  // 16-row MFMA blocks per wave
  static constexpr int kTN = BN / WN / 16;
  static constexpr int kChunksA = BM * (kBK / 16);  // 16-byte chunks per k-tile
  static constexpr int kChunksB = BN * (kBK / 16);
  static constexpr int kLoadsA = kChunksA / kThreads;
  static constexpr int kLoadsB = kChunksB / kThreads;
  static constexpr int kLdsBytes = 2 * (BM + BN) * kBK;
  static_assert(kChunksA % kThreads == 0 && kChunksB % kThreads == 0, "tile/threads");
};

// byte offset of 16-byte chunk c of row r inside a [rows][128 B] LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ (r & 7)) << 4); }

template <int OUT>
__device__ __forceinline__ void store4(void* C, int64_t idx, v4f v) {
  if constexpr (OUT == FP8SG_OUT_F32) {
    *reinterpret_cast<v4f*>(reinterpret_cast<float*>(C) + idx) = v;
  } else if constexpr (OUT == FP8SG_OUT_BF16) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<b4*>(reinterpret_cast<uint16_t*>(C) + idx) = h;
  } else {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<h4*>(reinterpret_cast<uint16_t*>(C) + idx) = h;
  }
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT>
__global__ __launch_bounds__(WM* WN* kWave) void k_gemm(GemmProblem p) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* As = smem;                  // [2][BM][128]
  uint8_t* Bs = smem + 2 * BM * kBK;   // [2][BN][128]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t bm = (int64_t)blockIdx.y * BM;
  const int64_t bn = (int64_t)blockIdx.x * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int nk = (int)((K + kBK - 1) / kBK);

  // global -> register prefetch of one k-tile
  uint4 ra[Cfg::kLoadsA], rb[Cfg::kLoadsB];
  auto load_tile = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      const int c = tid + i * Cfg::kThreads;
      const int r = c >> 3, kc = c & 7;
      const int64_t gr = bm + r, gk = k0 + 16 * kc;
      ra[i] = (gr < M && gk < K) ? *reinterpret_cast<const uint4*>(p.A + gr * K + gk)
                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      const int c = tid + i * Cfg::kThreads;
      const int r = c >> 3, kc = c & 7;
      const int64_t gr = bn + r, gk = k0 + 16 * kc;
      rb[i] = (gr < N && gk < K) ? *reinterpret_cast<const uint4*>(p.B + gr * K + gk)
                                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* a = As + buf * BM * kBK;
    uint8_t* b = Bs + buf * BN * kBK;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      const int c = tid + i * Cfg::kThreads;
      *reinterpret_cast<uint4*>(a + lds_off(c >> 3, c & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      const int c = tid + i * Cfg::kThreads;
      *reinterpret_cast<uint4*>(b + lds_off(c >> 3, c & 7)) = rb[i];
    }
  };

  v4f acc[Cfg::kTM][Cfg::kTN];
#pragma unroll
  for (int i = 0; i < Cfg::kTM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // fragment of a 16 x 128 block: lane holds row (lane & 15), K bytes
  // [32 * (lane >> 4), +32) as two 16-byte chunks.  A and B use the same K
  // mapping, so the products pair up correctly whatever order the
  // instruction sums them in.
  const int frow = lane & 15;
  const int fchunk = 2 * (lane >> 4);

  if (nk > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const uint8_t* a = As + buf * BM * kBK;
    const uint8_t* b = Bs + buf * BN * kBK;
    v8i bf[Cfg::kTN];
#pragma unroll
    for (int j = 0; j < Cfg::kTN; ++j) {
      const int r = wn * (BN / WN) + 16 * j + frow;
      const uint4 lo = *reinterpret_cast<const uint4*>(b + lds_off(r, fchunk));
      const uint4 hi = *reinterpret_cast<const uint4*>(b + lds_off(r, fchunk + 1));
      bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < Cfg::kTM; ++i) {
      const int r = wm * (BM / WM) + 16 * i + frow;
      const uint4 lo = *reinterpret_cast<const uint4*>(a + lds_off(r, fchunk));
      const uint4 hi = *reinterpret_cast<const uint4*>(a + lds_off(r, fchunk + 1));
      const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int j = 0; j < Cfg::kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], FB, FA,
                                                                     0, 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n..n+3] of each 16x16 block
  const float alpha = (float)(*p.inv_a * *p.inv_b);
#pragma unroll
  for (int i = 0; i < Cfg::kTM; ++i) {
    const int64_t m = bm + wm * (BM / WM) + 16 * i + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < Cfg::kTN; ++j) {
      const int64_t n = bn + wn * (BN / WN) + 16 * j + 4 * (lane >> 4);
      if (n >= N) continue;  // N % 16 == 0: the four columns are all in or all out
      v4f c = acc[i][j];
      c[0] *= alpha;
      c[1] *= alpha;
      c[2] *= alpha;
      c[3] *= alpha;
      store4<OUT>(p.C, m * N + n, c);
    }
  }
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT>
static hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  auto kern = k_gemm<BM, BN, WM, WN, FA, FB, OUT>;
  static bool attr_set = false;
  if (!attr_set && Cfg::kLdsBytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
  hipLaunchKernelGGL(kern, grid, dim3(Cfg::kThreads), Cfg::kLdsBytes, stream, p);
  return hipGetLastError();
}

template <int FA, int FB, int OUT>
static hipError_t launch_tiles(const GemmProblem& p, hipStream_t stream) {
  return launch_cfg<128, 128, 2, 2, FA, FB, OUT>(p, stream);
}

template <int FA, int FB>
static hipError_t launch_out(const GemmProblem& p, int out, hipStream_t stream) {
  switch (out) {
    case FP8SG_OUT_BF16: return launch_tiles<FA, FB, FP8SG_OUT_BF16>(p, stream);
    case FP8SG_OUT_F16: return launch_tiles<FA, FB, FP8SG_OUT_F16>(p, stream);
    default: return launch_tiles<FA, FB, FP8SG_OUT_F32>(p, stream);
  }
}

hipError_t launch_gemm(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E4M3FN) return launch_out<0, 0>(p, out, stream);
  if (fa == FP8SG_E5M2 && fb == FP8SG_E4M3FN) return launch_out<1, 0>(p, out, stream);
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E5M2) return launch_out<0, 1>(p, out, stream);
  return launch_out<1, 1>(p, out, stream);
}

}  // namespace fp8sg
