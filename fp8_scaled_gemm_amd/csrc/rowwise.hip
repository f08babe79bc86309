// Row-wise scaling [FP8-TRAIN §1: instead of one scale per tensor, each row
// has its own scale factor, which has to be carried through the
// accumulation].  For a GEMM C = A . B^T contracting over K, A gets one scale
// per row (over its K entries) and B one per row; both are constant along the
// contraction, so they factor out of the dot product and the epilogue applies
// alpha[m][n] = fl32(inv_a[m] * inv_b[n]) (gemm_rowwise.hip).  The backward
// GEMMs contract over the other dimension of each operand, so the transposed
// FP8 copy of a tensor is cast with one scale per column of the tensor (= per
// row of the copy): its codes differ from the row-major ones.
//
// Three kernels, two passes over x:
//   k_rw_amax:   per 128 x 128 tile, the maximum |x| of each of its rows
//                (DPP reductions over the row's 16 lanes) and of each of its
//                columns (shuffles, then LDS across the four waves), stored
//                as fp32 bits (NaN canonical) into partial-maximum arrays.  The arrays live in
//                the caller's q buffer, which the cast overwrites afterwards:
//                no workspace and no atomics.
//   k_rw_reduce: one lane per row (column): the maximum over its partials
//                (unsigned max of the bits: non-negative IEEE values order
//                like their bit patterns, NaN canonical above +inf), then the
//                amax and inverse-scale vectors.
//   k_rw_quant:  per tile, the 128 row scales and 128 column scales (fp64, as
//                for a tensor) into LDS; codes with the row scales stored
//                directly, codes with the column scales staged in LDS and
//                stored transposed.
// Passes that move 256 MiB or more load x with non-temporal loads; the code
// stores are non-temporal only once the codes alone are that large (16384^2
// with transposed copy: 313 -> 299 us for the three passes; 8192 x 14336,
// 235 MB of codes, is faster with cached stores: 120 against 135 us).
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kRwThreads = 256;
constexpr int kRwTile = 128;

// Partial maxima (fp32 bits) in the q buffer:
//   prow[ct * rows + r] = max |x[r, c]| over column tile ct
//   pcol[rt * cols + c] = max |x[r, c]| over row tile rt
// 4 (rows * tiles_c + cols * tiles_r) bytes <= rows * cols for rows, cols >= 16.
struct RwParts {
  uint32_t* prow;
  uint32_t* pcol;
};
__device__ __forceinline__ RwParts rw_parts(const RowwiseArgs& a) {
  uint32_t* base = reinterpret_cast<uint32_t*>(a.q);
  return {base, base + a.rows * a.tiles_c};
}
__host__ __device__ inline int64_t rw_tiles(int64_t n) { return (n + kRwTile - 1) / kRwTile; }

// One launch covers up to two tensors of the same kind (x and W of a layer):
// blocks [0, block0[1]) work on job 0, the rest on job 1.
struct RwJobs {
  RowwiseArgs job[2];
  int32_t block0[2];
  int32_t njobs;
};
__device__ __forceinline__ const RowwiseArgs& rw_job(const RwJobs& J, int64_t& b) {
  const int j = (J.njobs > 1 && (int)blockIdx.x >= J.block0[1]) ? 1 : 0;
  b = (int64_t)blockIdx.x - J.block0[j];
  return J.job[j];
}

// packed bf16 pair maximum (16-bit unsigned) -> the two fp32 bit patterns, NaN canonical
__device__ __forceinline__ void unpack_max(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = (d & 0xFFFFu) << 16;
  hi = d & 0xFFFF0000u;
  lo = lo > 0x7F800000u ? 0x7FC00000u : lo;
  hi = hi > 0x7F800000u ? 0x7FC00000u : hi;
}

template <bool WITH_T, bool S>
__global__ __launch_bounds__(kRwThreads) void k_rw_amax(RwJobs J) {
  int64_t b;
  const RowwiseArgs& a = rw_job(J, b);
  const int tid = threadIdx.x;
  const int64_t rows = a.rows, cols = a.cols;
  int64_t rt, ct;
  tile_grouped(b, rw_tiles(a.rows), a.tiles_c, rt, ct);
  const int64_t r_tile = rt * kRwTile, c_tile = ct * kRwTile;
  const RwParts pp = rw_parts(a);
  const int c8 = tid & 15, r0 = tid >> 4;
  const int64_t gc = c_tile + 8 * c8;
  const bool col_ok = gc < cols;  // cols % 16 == 0: a group of 8 is all in or all out
  __shared__ uint32_t srow[kRwTile];
  __shared__ uint4 red[kRwThreads / kWave][16];

  uint4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t gr = r_tile + r0 + 16 * p;
    v[p] = (col_ok && gr < rows) ? ld16<S>(a.x + gr * cols + gc) : make_uint4(0, 0, 0, 0);
  }
  constexpr uint32_t mask = 0x7FFF7FFFu;
  uint4 cm = make_uint4(0, 0, 0, 0);  // column maxima, two columns per dword
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    // this thread's 8 values of row r0 + 16p; the row's 16 lanes form one DPP row
    const uint32_t b = row16_max(absmax_bits(absmax8(0u, v[p])));
    if (c8 == 0) srow[r0 + 16 * p] = b;
    if constexpr (WITH_T) {
      cm.x = pmax(cm.x, v[p].x & mask);
      cm.y = pmax(cm.y, v[p].y & mask);
      cm.z = pmax(cm.z, v[p].z & mask);
      cm.w = pmax(cm.w, v[p].w & mask);
    }
  }
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  if constexpr (WITH_T) {
    // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same 8 columns
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
      cm.x = pmax(cm.x, (uint32_t)__shfl_xor((int)cm.x, off, kWave));
      cm.y = pmax(cm.y, (uint32_t)__shfl_xor((int)cm.y, off, kWave));
      cm.z = pmax(cm.z, (uint32_t)__shfl_xor((int)cm.z, off, kWave));
      cm.w = pmax(cm.w, (uint32_t)__shfl_xor((int)cm.w, off, kWave));
    }
    if (lane < 16) red[wave][lane] = cm;
  }
  __syncthreads();
  // the tile's 128 row maxima: 32 lanes, 4 consecutive rows each
  if (tid < kRwTile / 4) {
    const int64_t gr = r_tile + 4 * tid;
    if (gr < rows)  // rows % 16 == 0: four rows are all in or all out
      *reinterpret_cast<uint4*>(pp.prow + ct * rows + gr) =
          *reinterpret_cast<const uint4*>(&srow[4 * tid]);
  }
  if constexpr (WITH_T) {
    if (tid >= kWave && tid < kWave + 16) {
      const int c = tid - kWave;
      const int64_t gcc = c_tile + 8 * c;
      if (gcc < cols) {
        uint4 m = red[0][c];
#pragma unroll
        for (int w = 1; w < kRwThreads / kWave; ++w) {
          m.x = pmax(m.x, red[w][c].x);
          m.y = pmax(m.y, red[w][c].y);
          m.z = pmax(m.z, red[w][c].z);
          m.w = pmax(m.w, red[w][c].w);
        }
        uint4 o0, o1;
        unpack_max(m.x, o0.x, o0.y);
        unpack_max(m.y, o0.z, o0.w);
        unpack_max(m.z, o1.x, o1.y);
        unpack_max(m.w, o1.z, o1.w);
        uint32_t* dst = pp.pcol + rt * cols + gcc;
        *reinterpret_cast<uint4*>(dst) = o0;
        *reinterpret_cast<uint4*>(dst + 4) = o1;
      }
    }
  }
}

// One lane per row (then per column, with a transposed copy), 64 per block;
// the four waves split the partials and meet in LDS.
template <int FMT>
__global__ __launch_bounds__(kRwThreads) void k_rw_reduce(RwJobs J) {
  int64_t b;
  const RowwiseArgs& a = rw_job(J, b);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t rows = a.rows, ncols = a.qT ? a.cols : 0;
  const int64_t idx = b * kWave + lane;
  const RwParts pp = rw_parts(a);
  const bool is_row = idx < rows;
  const uint32_t* src = is_row ? pp.prow + idx : pp.pcol + (idx - rows);
  const int64_t stride = is_row ? rows : a.cols;
  const int64_t nt = idx < rows + ncols ? (is_row ? a.tiles_c : rw_tiles(rows)) : 0;
  constexpr int kWaves = kRwThreads / kWave;
  constexpr int kUnroll = 8;
  uint32_t m = 0;
  for (int64_t t0 = wave; t0 < nt; t0 += kWaves * kUnroll) {
    uint32_t u[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t t = t0 + (int64_t)kWaves * k;
      u[k] = t < nt ? src[t * stride] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) m = u[k] > m ? u[k] : m;
  }
  __shared__ uint32_t red[kWaves][kWave];
  red[wave][lane] = m;
  __syncthreads();
  if (wave == 0 && nt > 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = red[w][lane] > m ? red[w][lane] : m;
    const float amax = __uint_as_float(m);
    const double inv = scale_from_amax(amax, FMT).inv;
    if (is_row) {
      a.row_amax[idx] = amax;
      a.row_inv[idx] = inv;
    } else {
      a.col_amax[idx - rows] = amax;
      a.col_inv[idx - rows] = inv;
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

template <int FMT, bool WITH_T, bool S, bool SS>
__global__ __launch_bounds__(kRwThreads) void k_rw_quant(RwJobs J) {
  int64_t b;
  const RowwiseArgs& a = rw_job(J, b);
  const int tid = threadIdx.x;
  const int64_t rows = a.rows, cols = a.cols;
  // one block per tile; streaming with a transposed copy, XCD-contiguous order
  if constexpr (S && WITH_T) b = xcd_contiguous(b, rw_tiles(a.rows) * a.tiles_c);
  int64_t rt, ct;
  tile_grouped(b, rw_tiles(a.rows), a.tiles_c, rt, ct);
  const int64_t r_tile = rt * kRwTile, c_tile = ct * kRwTile;
  __shared__ float srow[kRwTile], scol[kRwTile];
  __shared__ uint32_t lds[kRwTile * 32];

  const int c8 = tid & 15, r0 = tid >> 4;
  const int64_t gc = c_tile + 8 * c8;
  const bool col_ok = gc < cols;
  uint4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t gr = r_tile + r0 + 16 * p;
    // branch-free: a lane outside a ragged tile loads x's first 8 elements;
    // their codes land only in rows and 16-row groups that are never stored
    v[p] = ld16<S>(a.x + ((col_ok && gr < rows) ? gr * cols + gc : 0));
  }
  if (tid < kRwTile) {
    const int64_t gr = r_tile + tid;
    srow[tid] = gr < rows ? scale_from_amax(a.row_amax[gr], FMT).s32 : 0.0f;
  } else if (WITH_T) {
    const int64_t gcc = c_tile + (tid - kRwTile);
    scol[tid - kRwTile] = gcc < cols ? scale_from_amax(a.col_amax[gcc], FMT).s32 : 0.0f;
  }
  __syncthreads();

  float sc[8];
  if constexpr (WITH_T) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] = scol[8 * c8 + j];
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = r0 + 16 * p;
    const int64_t gr = r_tile + r;
    if (col_ok && gr < rows) st8<SS>(a.q + gr * cols + gc, quant8<FMT>(v[p], srow[r]));
    if constexpr (WITH_T)
      *reinterpret_cast<uint2*>(&lds[r * 32 + ((2 * c8) ^ swz(r))]) = quant8v<FMT>(v[p], sc);
  }
  if constexpr (WITH_T) {
    __syncthreads();
    const int cq = tid >> 3, rq = tid & 7;
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * rq + i;
      d[i] = lds[r * 32 + (cq ^ swz(r))];
    }
    uint32_t o[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      tr4x4(d[4 * b], d[4 * b + 1], d[4 * b + 2], d[4 * b + 3], o[0][b], o[1][b], o[2][b], o[3][b]);
    const int64_t tr0 = r_tile + 16 * rq, tc0 = c_tile + 4 * cq;
    if (tr0 < rows && tc0 < cols) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st16<SS>(a.qT + (tc0 + j) * rows + tr0, make_uint4(o[j][0], o[j][1], o[j][2], o[j][3]));
    }
  }
}

// Blocks of a job: tiles for the amax and cast passes, 64 rows (columns) per
// block for the reduction.
static int64_t rw_tile_blocks(const RowwiseArgs& a) { return rw_tiles(a.rows) * a.tiles_c; }
static int64_t rw_reduce_blocks(const RowwiseArgs& a) {
  return (a.rows + (a.qT ? a.cols : 0) + kWave - 1) / kWave;
}

static RwJobs rw_jobs(const RowwiseArgs* a, int n, int64_t (*blocks)(const RowwiseArgs&),
                      int64_t& total) {
  RwJobs J{};
  J.njobs = n;
  total = 0;
  for (int j = 0; j < n; ++j) {
    J.job[j] = a[j];
    J.block0[j] = (int32_t)total;
    total += blocks(a[j]);
  }
  return J;
}

template <int FMT, bool S, bool WITH_T, bool SS = false>
static hipError_t launch_rw_passes(const RowwiseArgs* a, int n, hipStream_t stream) {
  int64_t nb, nred;
  const RwJobs Jt = rw_jobs(a, n, rw_tile_blocks, nb);
  const RwJobs Jr = rw_jobs(a, n, rw_reduce_blocks, nred);
  hipLaunchKernelGGL((k_rw_amax<WITH_T, S>), dim3((unsigned)nb), dim3(kRwThreads), 0, stream, Jt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rw_reduce<FMT>, dim3((unsigned)nred), dim3(kRwThreads), 0, stream, Jr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_rw_quant<FMT, WITH_T, S, SS>), dim3((unsigned)nb), dim3(kRwThreads), 0, stream,
                     Jt);
  return hipGetLastError();
}

// One or two non-empty casts with the same transposed-copy choice.
template <int FMT>
static hipError_t launch_rw_fmt(const RowwiseArgs* in, int n, hipStream_t stream) {
  RowwiseArgs a[2];
  int64_t bytes = 0;    // the cast's traffic
  int64_t written = 0;  // its codes
  for (int j = 0; j < n; ++j) {
    a[j] = in[j];
    a[j].tiles_c = (int32_t)rw_tiles(a[j].cols);
    // the partial maxima must fit in q (they do for rows, cols >= 16)
    const int64_t part_bytes =
        4 * (a[j].rows * a[j].tiles_c + (a[j].qT ? a[j].cols * rw_tiles(a[j].rows) : 0));
    if (part_bytes > a[j].rows * a[j].cols) return hipErrorInvalidValue;
    bytes += a[j].rows * a[j].cols * (a[j].qT ? 4 : 3);
    written += a[j].rows * a[j].cols * (a[j].qT ? 2 : 1);
  }
  const bool st = bytes >= kStreamBytes;
  if (a[0].qT && written >= kStreamBytes) return launch_rw_passes<FMT, true, true, true>(a, n, stream);
  if (a[0].qT) return st ? launch_rw_passes<FMT, true, true>(a, n, stream)
                         : launch_rw_passes<FMT, false, true>(a, n, stream);
  return st ? launch_rw_passes<FMT, true, false>(a, n, stream)
            : launch_rw_passes<FMT, false, false>(a, n, stream);
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
  return fmt == FP8SG_E4M3FN ? launch_rw_fmt<FP8SG_E4M3FN>(&a, 1, stream)
                             : launch_rw_fmt<FP8SG_E5M2>(&a, 1, stream);
}

hipError_t launch_rowwise2(const RowwiseArgs& a0, const RowwiseArgs& a1, int fmt,
                           hipStream_t stream) {
  // one grid must stay below 2^32 threads: at most 2^23 blocks of 256
  auto blocks = [](const RowwiseArgs& a) {
    const int64_t t = rw_tiles(a.rows) * rw_tiles(a.cols);
    const int64_t r = (a.rows + a.cols + kWave - 1) / kWave;
    return t > r ? t : r;
  };
  const bool together = a0.rows && a0.cols && a1.rows && a1.cols && !a0.qT == !a1.qT &&
                        blocks(a0) + blocks(a1) <= (int64_t(1) << 23);
  if (!together) {
    const hipError_t e = launch_rowwise(a0, fmt, stream);
    return e != hipSuccess ? e : launch_rowwise(a1, fmt, stream);
  }
  const RowwiseArgs a[2] = {a0, a1};
  return fmt == FP8SG_E4M3FN ? launch_rw_fmt<FP8SG_E4M3FN>(a, 2, stream)
                             : launch_rw_fmt<FP8SG_E5M2>(a, 2, stream);
}

}  // namespace fp8sg
