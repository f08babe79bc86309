// Row-wise scaling [FP8-TRAIN §1: instead of one scale per tensor, each row
// has its own scale factor, which has to be carried through the
// accumulation].  For a GEMM C = A . B^T contracting over K, A gets one scale
// per row (over its K entries) and B one per row; both are constant along the
// contraction, so they factor out of the dot product and the epilogue applies
// alpha[m][n] = fl32(inv_a[m] * inv_b[n]) (gemm.hip, ROWWISE epilogue).  The
// backward GEMMs contract over the other dimension of each operand, so the
// transposed FP8 copy of a tensor is cast with one scale per column of the
// tensor (= per row of the copy): its codes differ from the row-major ones.
//
// Two passes over x, as with per-tensor dynamic scaling:
//   k_rw_amax:  per 128 x 128 tile, the maximum |x| of each row (16-lane
//               shuffles) and of each column (shuffles, then LDS across the
//               four waves), merged into the caller's amax vectors with
//               unsigned atomic max on the fp32 bits (exact and order-free:
//               non-negative IEEE values order like their bit patterns, NaN
//               canonical above +inf).  The vectors start at zero (k_rw_zero).
//   k_rw_quant: per tile, the 128 row scales and 128 column scales (fp64, as
//               for a tensor) into LDS; codes with the row scales stored
//               directly, codes with the column scales staged in LDS and
//               stored transposed.  The blocks of the first tile column
//               (row) also write the row (column) inverse scales.
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kRwThreads = 256;
constexpr int kRwTile = 128;

__global__ __launch_bounds__(kRwThreads) void k_rw_zero(float* a, int64_t na, float* b, int64_t nb) {
  const int64_t i = (int64_t)blockIdx.x * kRwThreads + threadIdx.x;
  if (i < na) a[i] = 0.0f;
  if (b && i < nb) b[i] = 0.0f;
}

// the larger of the two bf16 magnitudes packed in m, as fp32 bits (NaN canonical)
__device__ __forceinline__ uint32_t pair_bits(uint32_t m) { return absmax_bits(m); }

template <bool WITH_T>
__global__ __launch_bounds__(kRwThreads) void k_rw_amax(RowwiseArgs a) {
  const int tid = threadIdx.x;
  const int64_t rows = a.rows, cols = a.cols;
  const int64_t r_tile = (int64_t)(blockIdx.x / a.tiles_c) * kRwTile;
  const int64_t c_tile = (int64_t)(blockIdx.x % a.tiles_c) * kRwTile;
  const int c8 = tid & 15, r0 = tid >> 4;
  const int64_t gc = c_tile + 8 * c8;
  const bool col_ok = gc < cols;  // cols % 16 == 0: a group of 8 is all in or all out
  constexpr uint32_t mask = 0x7FFF7FFFu;
  uint4 cm = make_uint4(0, 0, 0, 0);  // column maxima, two columns per dword
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t gr = r_tile + r0 + 16 * p;
    const uint4 v = (col_ok && gr < rows) ? *reinterpret_cast<const uint4*>(a.x + gr * cols + gc)
                                          : make_uint4(0, 0, 0, 0);
    uint32_t b = pair_bits(absmax8(0u, v));  // this thread's 8 values of row gr
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {  // the 16 lanes of a row are consecutive
      const uint32_t o = (uint32_t)__shfl_xor((int)b, off, kWave);
      b = o > b ? o : b;
    }
    if (c8 == 0 && gr < rows) atomicMax(reinterpret_cast<unsigned int*>(a.row_amax) + gr, b);
    if constexpr (WITH_T) {
      cm.x = pmax(cm.x, v.x & mask);
      cm.y = pmax(cm.y, v.y & mask);
      cm.z = pmax(cm.z, v.z & mask);
      cm.w = pmax(cm.w, v.w & mask);
    }
  }
  if constexpr (WITH_T) {
    // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same 8 columns
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
      cm.x = pmax(cm.x, (uint32_t)__shfl_xor((int)cm.x, off, kWave));
      cm.y = pmax(cm.y, (uint32_t)__shfl_xor((int)cm.y, off, kWave));
      cm.z = pmax(cm.z, (uint32_t)__shfl_xor((int)cm.z, off, kWave));
      cm.w = pmax(cm.w, (uint32_t)__shfl_xor((int)cm.w, off, kWave));
    }
    __shared__ uint4 red[kRwThreads / kWave][16];
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (lane < 16) red[wave][lane] = cm;
    __syncthreads();
    if (tid < 16 && col_ok) {
      uint4 m = red[0][tid];
#pragma unroll
      for (int w = 1; w < kRwThreads / kWave; ++w) {
        m.x = pmax(m.x, red[w][tid].x);
        m.y = pmax(m.y, red[w][tid].y);
        m.z = pmax(m.z, red[w][tid].z);
        m.w = pmax(m.w, red[w][tid].w);
      }
      unsigned int* ca = reinterpret_cast<unsigned int*>(a.col_amax) + gc;
      const uint32_t d[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lo = (d[k] & 0xFFFFu) << 16, hi = d[k] & 0xFFFF0000u;
        lo = lo > 0x7F800000u ? 0x7FC00000u : lo;
        hi = hi > 0x7F800000u ? 0x7FC00000u : hi;
        atomicMax(ca + 2 * k, lo);
        atomicMax(ca + 2 * k + 1, hi);
      }
    }
  }
}

// 8 bf16 values with 8 different scales (one per column) -> 8 codes
template <int FMT>
__device__ __forceinline__ uint2 quant8v(uint4 v, const float* s) {
  constexpr float m = FMT == FP8SG_E4M3FN ? kE4M3Max : kE5M2Max;
  float f0 = clamp_keep_nan(bf16_lo(v.x) * s[0], m), f1 = clamp_keep_nan(bf16_hi(v.x) * s[1], m);
  float f2 = clamp_keep_nan(bf16_lo(v.y) * s[2], m), f3 = clamp_keep_nan(bf16_hi(v.y) * s[3], m);
  float f4 = clamp_keep_nan(bf16_lo(v.z) * s[4], m), f5 = clamp_keep_nan(bf16_hi(v.z) * s[5], m);
  float f6 = clamp_keep_nan(bf16_lo(v.w) * s[6], m), f7 = clamp_keep_nan(bf16_hi(v.w) * s[7], m);
  return make_uint2(cvt4<FMT>(f0, f1, f2, f3), cvt4<FMT>(f4, f5, f6, f7));
}

// LDS tile for the transposed store: dword column x of row r at x ^ rw_swz(r)
__device__ __forceinline__ int rw_swz(int r) { return ((r >> 4) & 3) << 3; }

__device__ __forceinline__ void rw_tr4x4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                         uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  const uint32_t e0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
  const uint32_t e1 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
  const uint32_t f0 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
  const uint32_t f1 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
  o0 = __builtin_amdgcn_perm(f0, e0, 0x05040100u);
  o1 = __builtin_amdgcn_perm(f0, e0, 0x07060302u);
  o2 = __builtin_amdgcn_perm(f1, e1, 0x05040100u);
  o3 = __builtin_amdgcn_perm(f1, e1, 0x07060302u);
}

template <int FMT, bool WITH_T>
__global__ __launch_bounds__(kRwThreads) void k_rw_quant(RowwiseArgs a) {
  const int tid = threadIdx.x;
  const int64_t rows = a.rows, cols = a.cols;
  const int64_t r_tile = (int64_t)(blockIdx.x / a.tiles_c) * kRwTile;
  const int64_t c_tile = (int64_t)(blockIdx.x % a.tiles_c) * kRwTile;
  __shared__ float srow[kRwTile], scol[kRwTile];
  __shared__ uint32_t lds[kRwTile * 32];

  if (tid < kRwTile) {
    const int64_t gr = r_tile + tid;
    float s = 0.0f;
    if (gr < rows) {
      const ScaleVals sv = scale_from_amax(a.row_amax[gr], FMT);
      s = sv.s32;
      if (c_tile == 0) a.row_inv[gr] = sv.inv;
    }
    srow[tid] = s;
  } else if (WITH_T) {
    const int64_t gc = c_tile + (tid - kRwTile);
    float s = 0.0f;
    if (gc < cols) {
      const ScaleVals sv = scale_from_amax(a.col_amax[gc], FMT);
      s = sv.s32;
      if (r_tile == 0) a.col_inv[gc] = sv.inv;
    }
    scol[tid - kRwTile] = s;
  }
  __syncthreads();

  const int c8 = tid & 15, r0 = tid >> 4;
  const int64_t gc = c_tile + 8 * c8;
  const bool col_ok = gc < cols;
  float sc[8];
  if constexpr (WITH_T) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] = scol[8 * c8 + j];
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = r0 + 16 * p;
    const int64_t gr = r_tile + r;
    const uint4 v = (col_ok && gr < rows) ? *reinterpret_cast<const uint4*>(a.x + gr * cols + gc)
                                          : make_uint4(0, 0, 0, 0);
    if (col_ok && gr < rows)
      *reinterpret_cast<uint2*>(a.q + gr * cols + gc) = quant8<FMT>(v, srow[r]);
    if constexpr (WITH_T)
      *reinterpret_cast<uint2*>(&lds[r * 32 + ((2 * c8) ^ rw_swz(r))]) = quant8v<FMT>(v, sc);
  }
  if constexpr (WITH_T) {
    __syncthreads();
    const int cq = tid >> 3, rq = tid & 7;
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * rq + i;
      d[i] = lds[r * 32 + (cq ^ rw_swz(r))];
    }
    uint32_t o[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      rw_tr4x4(d[4 * b], d[4 * b + 1], d[4 * b + 2], d[4 * b + 3], o[0][b], o[1][b], o[2][b], o[3][b]);
    const int64_t tr0 = r_tile + 16 * rq, tc0 = c_tile + 4 * cq;
    if (tr0 < rows && tc0 < cols) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint4*>(a.qT + (tc0 + j) * rows + tr0) =
            make_uint4(o[j][0], o[j][1], o[j][2], o[j][3]);
    }
  }
}

template <int FMT>
static hipError_t launch_rw_fmt(RowwiseArgs a, hipStream_t stream) {
  const bool with_t = a.qT != nullptr;
  const int64_t nz = a.rows > a.cols ? a.rows : a.cols;
  hipLaunchKernelGGL(k_rw_zero, dim3((unsigned)((nz + kRwThreads - 1) / kRwThreads)), dim3(kRwThreads),
                     0, stream, a.row_amax, a.rows, with_t ? a.col_amax : nullptr, a.cols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.tiles_c = (int32_t)((a.cols + kRwTile - 1) / kRwTile);
  const int64_t nb = ((a.rows + kRwTile - 1) / kRwTile) * a.tiles_c;
  if (with_t) hipLaunchKernelGGL(k_rw_amax<true>, dim3((unsigned)nb), dim3(kRwThreads), 0, stream, a);
  else hipLaunchKernelGGL(k_rw_amax<false>, dim3((unsigned)nb), dim3(kRwThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (with_t)
    hipLaunchKernelGGL((k_rw_quant<FMT, true>), dim3((unsigned)nb), dim3(kRwThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((k_rw_quant<FMT, false>), dim3((unsigned)nb), dim3(kRwThreads), 0, stream, a);
  return hipGetLastError();
}

// An empty dimension: the other dimension's rows (columns) are empty, so
// their amax is 0 and their scale the one of amax 0.
template <int FMT>
__global__ __launch_bounds__(kRwThreads) void k_rw_empty(float* ra, double* ri, int64_t nr,
                                                         float* ca, double* ci, int64_t nc) {
  const int64_t i = (int64_t)blockIdx.x * kRwThreads + threadIdx.x;
  const double inv = scale_from_amax(0.0f, FMT).inv;
  if (i < nr) {
    ra[i] = 0.0f;
    ri[i] = inv;
  }
  if (ca && i < nc) {
    ca[i] = 0.0f;
    ci[i] = inv;
  }
}

template <int FMT>
static hipError_t launch_rw_empty(const RowwiseArgs& a, hipStream_t stream) {
  const bool with_t = a.qT != nullptr || a.col_amax != nullptr;
  const int64_t n = a.rows > a.cols ? a.rows : a.cols;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rw_empty<FMT>, dim3((unsigned)((n + kRwThreads - 1) / kRwThreads)),
                     dim3(kRwThreads), 0, stream, a.row_amax, a.row_inv, a.rows,
                     with_t ? a.col_amax : nullptr, a.col_inv, with_t ? a.cols : 0);
  return hipGetLastError();
}

hipError_t launch_rowwise(const RowwiseArgs& a, int fmt, hipStream_t stream) {
  if (a.rows == 0 || a.cols == 0)
    return fmt == FP8SG_E4M3FN ? launch_rw_empty<FP8SG_E4M3FN>(a, stream)
                               : launch_rw_empty<FP8SG_E5M2>(a, stream);
  return fmt == FP8SG_E4M3FN ? launch_rw_fmt<FP8SG_E4M3FN>(a, stream)
                             : launch_rw_fmt<FP8SG_E5M2>(a, stream);
}

}  // namespace fp8sg
