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
// Two kernels, one arithmetic: each wave issues v_mfma_f32_16x16x128_f8f6f4
// with the operand formats (e4m3 = 0, e5m2 = 1) selected per operand.  The B
// fragment is passed as the instruction's first source so each lane's four
// accumulators are four consecutive output columns.  LDS tiles hold 16-byte
// chunks XOR-swizzled by row so the fragment reads hit distinct banks.
//   - k_gemm_pingpong: 256 x 256 (or 224 x 256) tiles, for problems with at
//     least 128 of them (fills the chip).  A 16-bit output of kStreamOutBytes
//     or more is stored non-temporally.
//   - k_gemm: 128 x 128 tiles with register-staged loads, for smaller problems.
// Each kernel has a per-tensor epilogue (one alpha) and a row-wise one (RW:
// inverse-scale vectors along M and N); gemm.hip and gemm_rowwise.hip hold the
// two sets of instantiations.
#pragma once

#include <type_traits>

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
// A contraction-major k-tile row (one k, 128 output rows or columns) of the
// 128 x 128 kernel: the 16 lanes of a transposed read cover rows 8 apart
// (8 rows, 32 banks), and the four 16-lane groups rows 32 apart.  Bit 0 of
// the chunk swap follows bit 5 ^ bit 6 of the row, so any two groups that
// the LDS serves together fall on opposite bank sets.
__device__ __forceinline__ int lds_off_t(int r, int c) {
  return r * kBK + ((c ^ (r & 7) ^ (((r >> 5) ^ (r >> 6)) & 1)) << 4);
}

// The unscale step fused into an fp16 epilogue: the GradScaler's rounding
// sequence on the stored value, h = fp16(c), g = fp16(fl32(h) * inv_s), in
// packed conversions.  mx keeps the largest |g| bit pattern seen per 16-bit
// half; a half at 0x7C00 or above is inf/NaN (the standalone unscale pass's
// check on stored values).  Every element of the tile is checked, also rows
// and columns past M and N: their accumulators are exact zeros (the operand
// loads there are zero-filled), so they can only be non-finite when alpha
// is, and then every element in range is non-finite too.
struct Unscale {
  float inv_s;
  uint32_t mx;
  __device__ Unscale() : inv_s(0.f), mx(0u) {}
  __device__ void load(const GemmProblem& p) { inv_s = 1.0f / *p.amp_scale; }
  __device__ void set(float amp_scale) { inv_s = 1.0f / amp_scale; }
  // two elements: fp16 pair of fp16(fl32(fp16(c) * inv_s)), as packed bits
  __device__ uint32_t pair(f32x2 c) const {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 h = __builtin_convertvector(fp32_value(c), f16x2);
    const f32x2 u = __builtin_convertvector(h, f32x2);
    const f32x2 v = {u[0] * inv_s, u[1] * inv_s};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(fp32_value(v), f16x2));
  }
  __device__ uint2 apply(v4f c) {
    const uint2 r = make_uint2(pair(f32x2{c[0], c[1]}), pair(f32x2{c[2], c[3]}));
    mx = pmax(mx, pmax(r.x & 0x7FFF7FFFu, r.y & 0x7FFF7FFFu));
    return r;
  }
  // one plain store of 1 per wave that saw a non-finite value
  __device__ void flag(const GemmProblem& p, int lane) const {
    const bool bad = (mx & 0xFFFFu) >= 0x7C00u || (mx >> 16) >= 0x7C00u;
    if (__ballot(bad) != 0 && lane == 0) *p.found_inf = 1;
  }
};

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
    h4 h = {(_Float16)fp32_value(v[0]), (_Float16)fp32_value(v[1]), (_Float16)fp32_value(v[2]),
            (_Float16)fp32_value(v[3])};
    *reinterpret_cast<h4*>(reinterpret_cast<uint16_t*>(C) + idx) = h;
  }
}

// The epilogue factor.  Per-tensor scaling: alpha = fl32(inv_a * inv_b), one
// value [FP8-TRAIN §2].  Row-wise scaling (RW): inv_a and inv_b point to one
// inverse scale per row of A and of B, and element (m, n) is multiplied by
// fl32(inv_a[m] * inv_b[n]) [FP8-TRAIN §1: each row's scale is carried
// through the accumulation; constant along K, it factors out of the sum].
// A lane owns rows m0 + 16 i + (lane & 15) and columns n0 + 16 j + 4 (lane >> 4)
// + e of its wave's TM x TN blocks; the row-wise factors it needs are loaded
// once, after the main loop (rows and columns past M and N get 0, never stored).
template <bool RW, int TM, int TN>
struct Alpha {
  float a;
  double ia[RW ? TM : 1];
  double ib[RW ? TN : 1][4];
  __device__ Alpha(const GemmProblem& p, int64_t m0, int64_t n0, int lane) {
    if constexpr (RW) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + 16 * i + (lane & 15);
        ia[i] = m < p.M ? p.inv_a[m] : 0.0;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + 16 * j + 4 * (lane >> 4);  // N % 16 == 0: all four in or out
#pragma unroll
        for (int e = 0; e < 4; ++e) ib[j][e] = n < p.N ? p.inv_b[n + e] : 0.0;
      }
    } else {
      a = (float)(*p.inv_a * *p.inv_b);
    }
  }
  // per-tensor scaling with the two inverses given as values
  __device__ Alpha(double inv_a, double inv_b) {
    static_assert(!RW, "one factor");
    a = (float)(inv_a * inv_b);
  }
  // c holds C[m][n .. n+3] of block (i, j)
  __device__ void apply(v4f& c, int i, int j) const {
    if constexpr (RW) {
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] *= (float)(ia[i] * ib[j][e]);
    } else {
      c[0] *= a;
      c[1] *= a;
      c[2] *= a;
      c[3] *= a;
    }
  }
};

// The epilogue factor from inverse scales loaded earlier (per-tensor), or
// from the row-wise vectors in memory (RW).
template <bool RW, int TM, int TN>
__device__ __forceinline__ Alpha<RW, TM, TN> epilogue_alpha(const GemmProblem& p, int64_t m0, int64_t n0,
                                                        int lane, double inv_a, double inv_b) {
  if constexpr (RW) return Alpha<RW, TM, TN>(p, m0, n0, lane);
  else return Alpha<RW, TM, TN>(inv_a, inv_b);
}

// A bf16 operand cast to FP8 on its way into LDS (the small layers' one-launch
// passes, small_layer.hip): each 16-element chunk is quantized by quant8 at
// the tensor's scale32, the codes the cast kernels write; a block given `q`
// also stores its chunks' codes there, at the elements' own positions (the
// operand's stored layout).  x replaces the GEMM problem's code pointer.
struct CastSrc {
  const uint16_t* x;
  float s32;
  double inv;  // the tensor's inverse scale: the epilogue factor takes it
  uint8_t* q;
};

// Small-problem kernel: a BM x BN block tile per workgroup, K consumed 128
// bytes at a time.  Each k-tile of A and B is fetched with 16-byte global loads
// into registers while the previous tile is being multiplied, then written to
// the other half of a double-buffered LDS tile.  Each wave owns a (BM/WM) x
// (BN/WN) sub-tile of 16 x 16 blocks; results are stored as one 8-byte
// (bf16/fp16) or 16-byte (fp32) write per lane and block.
// TA / TB: the operand is stored contraction-major (A^T [K, M], B^T [K, N]);
// its k-tile is staged as 128 rows of 128 bytes (one per k, the tile's 128
// output rows or columns) and its fragments are read with ds_read_b64_tr_b8,
// as in the large-tile kernel below.
// CA / CB: the operand is a bf16 tensor cast on the fly (CastSrc ca / cb).
template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool RW, bool TA = false,
          bool TB = false, bool CA = false, bool CB = false>
__device__ __forceinline__ void gemm_small_tile(const GemmProblem& p, int bx, int by,
                                                CastSrc ca = CastSrc{}, CastSrc cb = CastSrc{}) {
  static_assert(!(TA || TB) || (BM == 128 && BN == 128), "contraction-major: 128 x 128 tiles");
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* As = smem;                  // [2][BM][128]
  uint8_t* Bs = smem + 2 * BM * kBK;   // [2][BN][128]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t bm = (int64_t)by * BM;
  const int64_t bn = (int64_t)bx * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int nk = (int)((K + kBK - 1) / kBK);

  // global -> register prefetch of one k-tile (a cast operand's chunk is 16
  // bf16 values, two 16-byte loads)
  uint4 ra[Cfg::kLoadsA * (CA ? 2 : 1)], rb[Cfg::kLoadsB * (CB ? 2 : 1)];
  // chunk c of a k-tile: LDS row c / 8, 16-byte chunk c % 8; a row-major
  // operand's row is an output row (column) and the chunk 16 k values, a
  // contraction-major one's row is a k and the chunk 16 output rows (columns).
  // The chunk's first element and whether it lies inside the operand:
  auto chunk_a = [&](int64_t k0, int c, int64_t& idx) {
    const int r = c >> 3, kc = c & 7;
    if constexpr (TA) {
      const int64_t gk = k0 + r, gm = bm + 16 * kc;
      idx = gk * M + gm;
      return gk < K && gm < M;
    } else {
      const int64_t gr = bm + r, gk = k0 + 16 * kc;
      idx = gr * K + gk;
      return gr < M && gk < K;
    }
  };
  auto chunk_b = [&](int64_t k0, int c, int64_t& idx) {
    const int r = c >> 3, kc = c & 7;
    if constexpr (TB) {
      const int64_t gk = k0 + r, gn = bn + 16 * kc;
      idx = gk * N + gn;
      return gk < K && gn < N;
    } else {
      const int64_t gr = bn + r, gk = k0 + 16 * kc;
      idx = gr * K + gk;
      return gr < N && gk < K;
    }
  };
  // (a value, not a named zero: a conditional between two lvalues would select
  // an address and put the zero in scratch memory)
  auto zero = []() { return make_uint4(0, 0, 0, 0); };
  auto load_tile = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      int64_t idx;
      const bool ok = chunk_a(k0, tid + i * Cfg::kThreads, idx);
      if constexpr (CA) {
        ra[2 * i] = ok ? *reinterpret_cast<const uint4*>(ca.x + idx) : zero();
        ra[2 * i + 1] = ok ? *reinterpret_cast<const uint4*>(ca.x + idx + 8) : zero();
      } else {
        ra[i] = ok ? *reinterpret_cast<const uint4*>(p.A + idx) : zero();
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      int64_t idx;
      const bool ok = chunk_b(k0, tid + i * Cfg::kThreads, idx);
      if constexpr (CB) {
        rb[2 * i] = ok ? *reinterpret_cast<const uint4*>(cb.x + idx) : zero();
        rb[2 * i + 1] = ok ? *reinterpret_cast<const uint4*>(cb.x + idx + 8) : zero();
      } else {
        rb[i] = ok ? *reinterpret_cast<const uint4*>(p.B + idx) : zero();
      }
    }
  };
  // a cast chunk's 16 codes (zero outside the operand, as the code loads
  // give); a block with a code buffer also stores them
  auto cast_chunk = [&](const CastSrc& cs, auto fmt, const uint4& lo, const uint4& hi, bool ok,
                        int64_t idx) {
    constexpr int F = decltype(fmt)::value;
    const uint2 a = quant8<F>(lo, cs.s32), b = quant8<F>(hi, cs.s32);
    const uint4 q = ok ? make_uint4(a.x, a.y, b.x, b.y) : zero();
    if (ok && cs.q) *reinterpret_cast<uint4*>(cs.q + idx) = q;
    return q;
  };
  auto store_tile = [&](int buf, int kt) {
    uint8_t* a = As + buf * BM * kBK;
    uint8_t* b = Bs + buf * BN * kBK;
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      const int c = tid + i * Cfg::kThreads;
      uint4 v;
      if constexpr (CA) {
        int64_t idx;
        const bool ok = chunk_a(k0, c, idx);
        v = cast_chunk(ca, std::integral_constant<int, FA>{}, ra[2 * i], ra[2 * i + 1], ok, idx);
      } else {
        v = ra[i];
      }
      *reinterpret_cast<uint4*>(a + (TA ? lds_off_t(c >> 3, c & 7) : lds_off(c >> 3, c & 7))) = v;
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      const int c = tid + i * Cfg::kThreads;
      uint4 v;
      if constexpr (CB) {
        int64_t idx;
        const bool ok = chunk_b(k0, c, idx);
        v = cast_chunk(cb, std::integral_constant<int, FB>{}, rb[2 * i], rb[2 * i + 1], ok, idx);
      } else {
        v = rb[i];
      }
      *reinterpret_cast<uint4*>(b + (TB ? lds_off_t(c >> 3, c & 7) : lds_off(c >> 3, c & 7))) = v;
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
  // fragment of output block blk from a contraction-major k-tile (128 rows
  // of 128 B): four transposed 8-byte reads
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  auto frag_t = [&](const uint8_t* base, int blk) {
    v8i out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 32 * (lane >> 4) + 8 * r + (frow >> 1);
      const v2i_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i_t*)(base + lds_off_t(row, blk) + 8 * (frow & 1)));
      out[2 * r] = t.x;
      out[2 * r + 1] = t.y;
    }
    return out;
  };

  if (nk > 0) {
    load_tile(0);
    store_tile(0, 0);
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
      if constexpr (TB) {
        bf[j] = frag_t(b, wn * (BN / WN) / 16 + j);
      } else {
        const int r = wn * (BN / WN) + 16 * j + frow;
        const uint4 lo = *reinterpret_cast<const uint4*>(b + lds_off(r, fchunk));
        const uint4 hi = *reinterpret_cast<const uint4*>(b + lds_off(r, fchunk + 1));
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::kTM; ++i) {
      v8i af;
      if constexpr (TA) {
        af = frag_t(a, wm * (BM / WM) / 16 + i);
      } else {
        const int r = wm * (BM / WM) + 16 * i + frow;
        const uint4 lo = *reinterpret_cast<const uint4*>(a + lds_off(r, fchunk));
        const uint4 hi = *reinterpret_cast<const uint4*>(a + lds_off(r, fchunk + 1));
        af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < Cfg::kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], FB, FA,
                                                                     0, 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1, kt + 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n..n+3] of each 16x16 block; a cast operand
  // brings its inverse scale as a value
  auto make_alpha = [&]() {
    if constexpr (CA || CB)
      return Alpha<RW, Cfg::kTM, Cfg::kTN>(CA ? ca.inv : *p.inv_a, CB ? cb.inv : *p.inv_b);
    else
      return Alpha<RW, Cfg::kTM, Cfg::kTN>(p, bm + wm * (BM / WM), bn + wn * (BN / WN), lane);
  };
  const Alpha<RW, Cfg::kTM, Cfg::kTN> alpha = make_alpha();
  Unscale us;
  if constexpr (OUT == kOutF16Unscale) us.load(p);
#pragma unroll
  for (int i = 0; i < Cfg::kTM; ++i) {
    const int64_t m = bm + wm * (BM / WM) + 16 * i + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < Cfg::kTN; ++j) {
      const int64_t n = bn + wn * (BN / WN) + 16 * j + 4 * (lane >> 4);
      if (n >= N) continue;  // N % 16 == 0: the four columns are all in or all out
      v4f c = acc[i][j];
      alpha.apply(c, i, j);
      if constexpr (OUT == kOutF16Unscale)
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + m * N + n) = us.apply(c);
      else
        store4<OUT>(p.C, m * N + n, c);
    }
  }
  if constexpr (OUT == kOutF16Unscale) us.flag(p, lane);
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool RW, bool TA = false,
          bool TB = false>
__global__ __launch_bounds__(WM* WN* kWave) void k_gemm(GemmProblem p) {
  gemm_small_tile<BM, BN, WM, WN, FA, FB, OUT, RW, TA, TB>(p, blockIdx.x, blockIdx.y);
}

// Two independent small problems of the same kind in one launch (the small
// backward pass's dgrad and wgrad, where launches dominate): blockIdx.z picks
// the problem; blocks past its tiles leave at once.
template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool RW, bool TA0 = false,
          bool TB0 = false, bool TA1 = false, bool TB1 = false>
__global__ __launch_bounds__(WM* WN* kWave) void k_gemm2(GemmProblem p0, GemmProblem p1) {
  const GemmProblem& p = blockIdx.z ? p1 : p0;
  if ((int64_t)blockIdx.y * BM >= p.M || (int64_t)blockIdx.x * BN >= p.N) return;
  if constexpr (TA0 == TA1 && TB0 == TB1) {
    gemm_small_tile<BM, BN, WM, WN, FA, FB, OUT, RW, TA0, TB0>(p, blockIdx.x, blockIdx.y);
  } else {
    if (blockIdx.z)
      gemm_small_tile<BM, BN, WM, WN, FA, FB, OUT, RW, TA1, TB1>(p, blockIdx.x, blockIdx.y);
    else
      gemm_small_tile<BM, BN, WM, WN, FA, FB, OUT, RW, TA0, TB0>(p, blockIdx.x, blockIdx.y);
  }
}

// ---------------------------------------------------------------------------
// Large-tile kernel helpers.  Operand tiles are streamed global -> LDS by the
// buffer unit (buffer_load_dwordx4 ... lds), with no VGPR staging.  One load
// instruction moves 64 lanes x 16 B = 1 KB = 8 rows of a 128-byte k-slice;
// lane l fills LDS row 8g + l/8, chunk l%8, and fetches the global chunk that
// belongs there under the swizzle.  The per-block buffer descriptor spans only
// the block's row panel, so rows past M (or N) read as zero; chunks past K are
// pointed outside the descriptor and read as zero too.
// ---------------------------------------------------------------------------

// 16-byte chunk c of LDS row r lives at chunk c ^ swz16(r).  swz16 is a
// bijection on every aligned group of 8 rows and on the even and the odd rows
// of every aligned group of 16, so the 16-byte fragment reads hit distinct
// banks whether the LDS serves 8 lanes x 16 B or 16 lanes x 16 B per cycle.
// It depends on r & 15 only, so a lane's fragment-read address differs
// between 16-row blocks by a constant that fits the instruction's offset.
__device__ __forceinline__ int swz16(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
__device__ __forceinline__ int lds_off2(int r, int c) { return r * kBK + ((c ^ swz16(r)) << 4); }

// s_waitcnt with vmcnt <= n and the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, gfx9 data format
constexpr uint32_t kOob = 0x80000000u;        // offset past any descriptor: reads 0

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes), in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = (int)kBufDword3;
  return r;
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds + 16 * lane.
// Written as inline assembly so the compiler does not track these LDS writes:
// its own wait insertion would otherwise drain every in-flight load before each
// LDS read.  The k-loop below waits for them explicitly (s_waitcnt vmcnt) and
// orders LDS reads with compiler barriers.  M0 carries the LDS address; no
// other code in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// The same with the offset split into a per-lane part and a wave-uniform
// part, added inside the statement: the sum lives only here, so the compiler
// keeps no per-load offset registers across the k-loop.  vbase + sbase stays
// below 2^32 (vbase < 2^31, sbase <= kOob).
__device__ __forceinline__ void lds_dma16_split(uint32_t lds, uint32_t vbase, uint32_t sbase, i32x4 rsrc) {
  uint32_t tmp;
  asm volatile("v_add_u32 %0, %1, %2\n\ts_mov_b32 m0, %3\n\ts_nop 1\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
               : "=&v"(tmp)
               : "s"(sbase), "v"(vbase), "s"(lds), "s"(rsrc)
               : "memory", "m0");
}

#pragma clang diagnostic pop

// LDS byte address of a __shared__ array (folds to a constant).
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Position of this block's tile.  Workgroups are handed to the 8 XCDs round
// robin (block b on XCD b % 8); renumber so that each XCD gets a run of
// consecutive tile indices, then walk tiles in groups of kGroupM tile-rows,
// column by column, so one XCD's tiles form a compact region whose A and B
// panels its L2 can share.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_of_index(int b, int nbm, int nbn, int& tm, int& tn) {
  const int nb = nbm * nbn;
  const int q = nb / 8, rem = nb % 8, x = b % 8;
  const int t = x * q + (x < rem ? x : rem) + b / 8;
  const int per_group = kGroupM * nbn;
  const int g = t / per_group, r = t % per_group;
  const int gm = (nbm - g * kGroupM) < kGroupM ? (nbm - g * kGroupM) : kGroupM;
  tm = g * kGroupM + r % gm;
  tn = r / gm;
}
__device__ __forceinline__ void tile_of(int nbm, int nbn, int& tm, int& tn) {
  tile_of_index(blockIdx.x, nbm, nbn, tm, tn);
}

// ---------------------------------------------------------------------------
// Large-tile kernel: BM x 256 output tile per workgroup, K consumed 128 bytes
// at a time, 8 waves in two groups of four (one wave of each group per SIMD).
// Group g owns output rows [BM/2 g, BM/2 (g + 1)); wave q of a group owns
// columns [64 q, 64 q + 64), i.e. BM/32 x 4 blocks of 16 x 16.
//
// The groups run half a k-tile apart and alternate between
//   - a memory phase: issue this group's share of the global -> LDS loads,
//     then read all 12 operand fragments of the next k-tile (8 A, 4 B; 96
//     VGPRs) from LDS, and
//   - a compute phase: 32 MFMAs on registers only, nothing to wait for,
// meeting at a workgroup barrier at every swap.  So each SIMD always has one
// wave feeding its matrix pipe while the other waits on LDS and memory.
//
// LDS (160 KB): A of k-tile t in A stage t % 2, B of k-tile t in B slot
// t % 3.  Group 0 loads A of t + 1 during its memory phase for t (that stage
// held A of t - 1, which both groups read before the last swap); group 1
// loads B of t + 2 during its memory phase for t (that slot held B of t - 1).
// Each load is waited for (s_waitcnt vmcnt) by the wave that issued it before
// the swap ahead of the first read, so the barrier publishes it to all waves.
// ---------------------------------------------------------------------------
//
// BM is 256 or 224.  A 224-row tile (7 blocks of 16 rows per wave group) fits
// M = 14336 in exactly 64 tile rows: the MLP block's weight-gradient GEMMs then
// have 1024 tiles, four rounds over 256 CUs with none idle, instead of 896
// (the last of four rounds half empty).  The launcher picks it by that count.
//
// TR (transposed roles): the launcher swaps the operands, so the kernel forms
// C^T = B A^T with 224-row tiles along the original N (p.M and p.N are the
// original N and M, p.A and p.B the original B and A) and writes C itself:
// the MFMA takes the A-slot fragment first, so a lane's four accumulators are
// again four consecutive columns of C, and the epilogue stages each tile
// transposed.  That fits N = 14336 in 64 tiles when M = 4096 does not fit 224
// (the MLP block's down-projection weight gradient: 1024 tiles, four full
// rounds, instead of 896 tiles of 256 x 256).
// ---------------------------------------------------------------------------
//
// TA / TB (operands stored contraction-major): A is given as A^T [K, M] (or B
// as B^T [K, N]) row-major, i.e. the FP8 codes of a tensor in its own layout
// where the GEMM contracts over its rows -- the backward GEMMs' operands,
// without a transposed copy.  Such an operand's k-tile is staged as 128 LDS
// rows (one per k) of 256 bytes (the tile's output rows or columns), 16-byte
// chunk q of row r at position q ^ swzT(r), and each fragment is gathered
// with four ds_read_b64_tr_b8: in every group of 16 lanes the 8-byte reads
// of lanes 2i and 2i + 1 form row i of an 8 x 16 byte matrix and lane j
// receives its column j, so lane j of group g, pointing at row
// 32 g + 8 r + j / 2, chunk half j & 1, receives k = 32 g + 8 r .. + 7 of its
// output row or column.  Rows past K fall outside the buffer descriptor and
// read as zero (no ragged-K test); columns past M or N are pointed outside.
// swzT(r) = (r & 7) | 8 ((r >> 5 ^ r >> 6) & 1): the 16 lanes of a group read
// 8 rows at 8 chunk positions, one 128-byte half of the 64 banks, and the
// four groups rows 32 apart; the bit-3 term puts any two groups that the LDS
// serves together (0 and 1 or 0 and 2, 2 and 3 or 1 and 3) in opposite halves
// (without it every transposed read took a two-way bank conflict).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swzT(int r) { return (r & 7) | ((((r >> 5) ^ (r >> 6)) & 1) << 3); }

template <int FA, int FB, int OUT, bool RAGGED_K, bool RW, int BM = 256, bool TR = false,
          bool TA = false, bool TB = false>
__global__ __launch_bounds__(512) void k_gemm_pingpong(GemmProblem p) {
  static_assert(BM == 256 || BM == 224, "tile rows");
  static_assert(!(TR && RW), "transposed roles: per-tensor scaling only");
  static_assert(!(RW && (TA || TB)), "contraction-major operands: per-tensor scaling only");
  constexpr int BN = 256;
  constexpr int kTM = BM / 32, kTN = 4;
  constexpr int kLoads = 256 / 8 / 4;  // 1 KB loads per group wave per B stage: 8
  constexpr int kLoadsA = BM / 32;     // ... per A stage: 8, or 7 at BM = 224
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[256 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[256 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[256 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[256 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[256 * kBK];
  auto sa = [&](auto i) -> uint8_t* { if constexpr (decltype(i)::value == 0) return sA0; else return sA1; };
  auto sb = [&](auto i) -> uint8_t* {
    constexpr int I = decltype(i)::value;
    if constexpr (I == 0) return sB0;
    else if constexpr (I == 1) return sB1;
    else return sB2;
  };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int grp = wave >> 2, wq = wave & 3;
  const int64_t M = p.M, N = p.N, K = p.K;
  // The epilogue's inputs from memory (per-tensor inverse scales, the loss
  // scale), loaded before the main loop: loaded after it, every tile's
  // epilogue waited one memory round trip for them.  Uniform, so they stay
  // in scalar registers through the loop.
  double inv_a0 = 0.0, inv_b0 = 0.0;
  float amp0 = 1.0f;
  if constexpr (!RW) {
    inv_a0 = *p.inv_a;
    inv_b0 = *p.inv_b;
  }
  if constexpr (OUT == kOutF16Unscale) amp0 = *p.amp_scale;
  const int nbm = (int)((M + BM - 1) / BM), nbn = (int)((N + BN - 1) / BN);
  int tm, tn;
  tile_of(nbm, nbn, tm, tn);
  const int64_t bm = (int64_t)tm * BM, bn = (int64_t)tn * BN;
  const int nk = (int)((K + kBK - 1) / kBK);
  const int64_t rows_a = (M - bm) < BM ? (M - bm) : BM;
  const int64_t rows_b = (N - bn) < BN ? (N - bn) : BN;
  // a contraction-major operand's descriptor starts at the tile's first
  // column and ends with row K - 1
  const i32x4 ra = TA ? make_rsrc(p.A + bm, K * M - bm) : make_rsrc(p.A + bm * K, rows_a * K);
  const i32x4 rb = TB ? make_rsrc(p.B + bn, K * N - bn) : make_rsrc(p.B + bn * K, rows_b * K);

  // One operand stage (BM or 256 rows x 128 B) by wave q of a group: rows
  // [8 L q, 8 L q + 8 L), L loads of 8 rows (L = 8 for B, BM / 32 for A).
  // Lane l of load i fills LDS row 8 (L q + i) + l / 8; the swizzle of that row
  // depends only on (L q + i) & 1, so a lane needs two offsets (even and odd)
  // and the rest is scalar.  Only a ragged last k-tile (RAGGED_K) needs the
  // per-lane test against K.
  const int lr = lane >> 3;
  const int cl0 = (lane & 7) ^ swz16(lr), cl1 = (lane & 7) ^ swz16(8 + lr);
  const uint32_t vo0 = (uint32_t)(lr * K + 16 * cl0), vo1 = (uint32_t)(lr * K + 16 * cl1);
  auto issue = [&](auto nl, int kt, uint32_t dst, const i32x4& rs) {  // kt >= nk loads zeros
    constexpr int L = decltype(nl)::value;
    const int k0 = kt < nk ? kt * kBK : (int)K;
    const uint32_t sbase = (uint32_t)(8 * L * wq * K + k0);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool odd = (L % 2 == 0 ? i : wq + i) & 1;  // (L q + i) & 1
      uint32_t off = (odd ? vo1 : vo0) + sbase + (uint32_t)(8 * i * K);
      if constexpr (RAGGED_K) {
        if (k0 + 16 * (odd ? cl1 : cl0) >= K) off = kOob;
      } else {
        if (kt >= nk) off = kOob;
      }
      lds_dma16(dst + (wq * L + i) * 1024, off, rs);
    }
  };
  // A contraction-major operand's stage (128 rows of 256 B) by wave q of a
  // group: 8 loads of 4 rows, rows 32 q + 4 i + l / 16, LDS position l % 16;
  // the row's swizzle swzT(32 q + 4 i + l / 16) takes two values per lane (i
  // even or odd), so a lane needs two offsets and the rest is scalar.  `ld` is
  // the stored row length (M or N), `ncols` that of the tile's columns left.
  const int lr4 = lane >> 4, lp = lane & 15;
  auto t_off = [&](int row, int64_t ld, int64_t ncols) -> uint32_t {
    const int q = lp ^ swzT(row);
    return 16 * q < ncols ? (uint32_t)(lr4 * ld + 16 * q) : 0x7FFFFFF0u;
  };
  const int trow = 32 * wq + lr4;
  const uint32_t ta0 = TA ? t_off(trow, M, M - bm) : 0u, ta1 = TA ? t_off(trow + 4, M, M - bm) : 0u;
  const uint32_t tb0 = TB ? t_off(trow, N, N - bn) : 0u, tb1 = TB ? t_off(trow + 4, N, N - bn) : 0u;
  // A load's 4 rows lie all below K or all past it (K is a multiple of 16):
  // load i is in range while 4 i < K - (128 kt + 32 q); past K its scalar part
  // is the outside offset, so no row offset exceeds (K - 4) ld < 2^31.  All of
  // it is 32-bit scalar arithmetic (K, M and N are below 2^31), the row
  // offset stepped by 4 ld from load to load; 4 ld passes through an empty
  // asm statement so the compiler does not hoist the eight multiples out of
  // the k-loop (they spilled scalar registers).
  const int K32 = (int)K;
  auto issue_t = [&](int kt, uint32_t dst, const i32x4& rs, uint32_t ld, uint32_t v0, uint32_t v1) {
    const int r0 = kt * kBK + 32 * wq;
    const int rem = kt < nk ? K32 - r0 : 0;
    uint32_t ld4 = 4 * ld;
    asm volatile("" : "+s"(ld4));
    uint32_t sb = (uint32_t)r0 * ld;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds_dma16_split(dst + (wq * 8 + i) * 1024, (i & 1) ? v1 : v0, 4 * i < rem ? sb : kOob, rs);
      sb += ld4;
    }
  };
  using LA = std::integral_constant<int, TA ? 8 : kLoadsA>;
  using LB = std::integral_constant<int, kLoads>;
  // this group's loads of operand A (group 0) or B (group 1) for k-tile kt
  auto issue_a = [&](int kt, uint32_t dst) {
    if constexpr (TA) issue_t(kt, dst, ra, (uint32_t)M, ta0, ta1);
    else issue(LA{}, kt, dst, ra);
  };
  auto issue_b = [&](int kt, uint32_t dst) {
    if constexpr (TB) issue_t(kt, dst, rb, (uint32_t)N, tb0, tb1);
    else issue(LB{}, kt, dst, rb);
  };
  v4f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fchunk = 2 * (lane >> 4);
  auto frag = [&](const uint8_t* base, int blk) {
    const int r = 16 * blk + frow;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + lds_off2(r, fchunk));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + lds_off2(r, fchunk + 1));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // fragment of output block blk (16 rows or columns) from a contraction-major
  // stage: four transposed 8-byte reads (see above).  The lane reads rows
  // 32 g + 8 r + lp / 2, all with swizzle swzT(32 g + lp / 2), so its
  // addresses are t_base + r * 2048 + ((blk ^ swzT(..)) << 4).  The XOR
  // differs per block and lane; `sx` (swzT(..) << 4) is passed through an
  // empty asm statement once per memory phase so the compiler recomputes the
  // XORs there instead of keeping one address register per block live across
  // the k-loop.
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  const uint32_t t_base = (uint32_t)((32 * lr4 + (lp >> 1)) * 256 + 8 * (lp & 1));
  auto frag_t = [&](const uint8_t* base, int blk, uint32_t sx) {
    v8i out;
    const uint32_t a0 = lds_u32(base) + t_base + (((uint32_t)blk << 4) ^ sx);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v2i_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i_t*)(uintptr_t)(a0 + 2048 * r));
      out[2 * r] = t.x;
      out[2 * r + 1] = t.y;
    }
    return out;
  };
  const int ra0 = grp * kTM, rb0 = wq * 4;
  v8i af[kTM], bf[kTN];
  auto barrier = [&]() {
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

  // Prologue: group 0 loads A0, group 1 loads B0 and B1.
  if (grp == 0) {
    issue_a(0, lds_u32(sA0));
    wait_vmcnt<0>();
  } else {
    issue_b(0, lds_u32(sB0));
    issue_b(1, lds_u32(sB1));
    wait_vmcnt<kLoads>();
  }
  barrier();
  if (grp == 1) barrier();  // group 1 starts half a k-tile later

  // k-tile t: memory phase (loads, then all 12 fragments), swap, compute
  // phase, swap.  Group 0 loads A of t + 1 (its stage held A of t - 1, read
  // by both groups before the last swap) and waits for it before the swap
  // that ends its compute phase.  Group 1 loads B of t + 2 (its slot held B
  // of t - 1) and, before the swap that ends this memory phase, waits for B of
  // t + 1, issued one k-tile earlier.
  auto step = [&](auto pc, int t) {
    constexpr int P = decltype(pc)::value;  // t % 6
    const uint8_t* a = sa(std::integral_constant<int, P % 2>{});
    const uint8_t* b = sb(std::integral_constant<int, P % 3>{});
    {
      const uint32_t da = lds_u32(sa(std::integral_constant<int, (P + 1) % 2>{}));
      const uint32_t db = lds_u32(sb(std::integral_constant<int, (P + 2) % 3>{}));
      if constexpr (LA::value == kLoads && TA == TB) {
        if constexpr (TA) issue_t(t + 1 + grp, grp ? db : da, grp ? rb : ra, (uint32_t)(grp ? N : M),
                                  grp ? tb0 : ta0, grp ? tb1 : ta1);
        else issue(LB{}, t + 1 + grp, grp ? db : da, grp ? rb : ra);
      } else {
        if (grp) issue_b(t + 2, db);
        else issue_a(t + 1, da);
      }
    }
    uint32_t sx = (uint32_t)swzT(32 * lr4 + (lp >> 1)) << 4;
    if constexpr (TA || TB) asm volatile("" : "+v"(sx));
#pragma unroll
    for (int j = 0; j < kTN; ++j) bf[j] = TB ? frag_t(b, rb0 + j, sx) : frag(b, rb0 + j);
#pragma unroll
    for (int i = 0; i < kTM; ++i) af[i] = TA ? frag_t(a, ra0 + i, sx) : frag(a, ra0 + i);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (grp == 1) wait_vmcnt<kLoads>();  // B of t + 1 has landed
    barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = TR ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], FA,
                                                                          FB, 0, 0, 0, 0)
                       : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], FB,
                                                                          FA, 0, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) wait_vmcnt<0>();  // A of t + 1 has landed
    barrier();
  };
  // The launcher sends Kc == 0 to the small kernel.  Should an empty
  // contraction arrive here anyway, the >= test ends the loop after one step
  // over k-tile 0, whose loads all lie past K and read as zeros.  (This loop
  // shape keeps the accumulators in registers; a test at the top of the loop,
  // or a branch around it, made the compiler spill them.)
  for (int t = 0;;) {
    step(std::integral_constant<int, 0>{}, t);
    if (++t >= nk) break;
    step(std::integral_constant<int, 1>{}, t);
    if (++t >= nk) break;
    step(std::integral_constant<int, 2>{}, t);
    if (++t >= nk) break;
    step(std::integral_constant<int, 3>{}, t);
    if (++t >= nk) break;
    step(std::integral_constant<int, 4>{}, t);
    if (++t >= nk) break;
    step(std::integral_constant<int, 5>{}, t);
    if (++t >= nk) break;
  }
  if (grp == 0) barrier();

  const int wr0 = grp * (BM / 2), wc0 = wq * 64;
  const Alpha<RW, kTM, kTN> alpha = epilogue_alpha<RW, kTM, kTN>(p, bm + wr0, bn + wc0, lane, inv_a0, inv_b0);
  // Block (i, j) of this lane, in the C tile: row r, columns col .. col + 3.
  // The C tile is BM x 256 (rows along p.M), or 256 x BM under TR (rows along
  // p.N, which is then the original M); C's rows are c_rows long.
  auto tile_rc = [&](int i, int j, int& r, int& col) {
    if constexpr (TR) {
      r = wc0 + 16 * j + (lane & 15);
      col = wr0 + 16 * i + 4 * (lane >> 4);
    } else {
      r = wr0 + 16 * i + (lane & 15);
      col = wc0 + 16 * j + 4 * (lane >> 4);
    }
  };
  const int64_t c_rows = TR ? N : M, c_cols = TR ? M : N;
  const int64_t row0 = TR ? bn : bm, col0 = TR ? bm : bn;
  if constexpr (OUT == FP8SG_OUT_F32) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        int r, col;
        tile_rc(i, j, r, col);
        const int64_t m = row0 + r, n = col0 + col;
        if (m >= c_rows || n >= c_cols) continue;
        v4f c = acc[i][j];
        alpha.apply(c, i, j);
        store4<OUT>(p.C, m * c_cols + n, c);
      }
    }
  } else {
    constexpr int kRowBytes = 2 * BN;
    auto crow = [&](int r) -> uint8_t* {
      uint8_t* base = r < 64 ? sA0 : r < 128 ? sA1 : r < 192 ? sB0 : sB1;
      return base + (r & 63) * kRowBytes;
    };
    Unscale us;
    if constexpr (OUT == kOutF16Unscale) us.set(amp0);
    __builtin_amdgcn_s_waitcnt(0);  // no load may still be writing a slot
    barrier();
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        int r, col;
        tile_rc(i, j, r, col);
        v4f c = acc[i][j];
        alpha.apply(c, i, j);
        const int off = (((col >> 3) ^ (r & 31)) << 4) + (col & 7) * 2;
        if constexpr (OUT == kOutF16Unscale)
          *reinterpret_cast<uint2*>(crow(r) + off) = us.apply(c);
        else
          store4<OUT>(crow(r) + off, 0, c);
      }
    }
    if constexpr (OUT == kOutF16Unscale) us.flag(p, lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier();
    // the staged tile, 16-byte chunks of 8 columns: BM rows x 32 chunks, or
    // under TR 256 rows x BM / 8 chunks (28 at BM = 224)
    constexpr int kChunks = TR ? BM / 8 : BN / 8;
    auto write_tile = [&](auto nt) {
#pragma unroll
      for (int pass = 0; pass < BM / 16; ++pass) {
        const int id = pass * 512 + (int)threadIdx.x;
        const int r = id / kChunks, cc = id % kChunks;
        const uint4 v = *reinterpret_cast<const uint4*>(crow(r) + ((cc ^ (r & 31)) << 4));
        const int64_t m = row0 + r, n = col0 + 8 * cc;
        if (m < c_rows && n < c_cols) st16<decltype(nt)::value>(reinterpret_cast<uint16_t*>(p.C) + m * c_cols + n, v);
      }
    };
    if (2 * c_rows * c_cols >= kStreamOutBytes) write_tile(std::true_type{});
    else write_tile(std::false_type{});
  }
}

// TR: p is the problem with its operands swapped (see k_gemm_pingpong).
template <int FA, int FB, int OUT, bool RW, int BM, bool TR = false, bool TA = false, bool TB = false>
static hipError_t launch_pingpong(const GemmProblem& p, hipStream_t stream) {
  const unsigned nb = (unsigned)(((p.M + BM - 1) / BM) * ((p.N + 255) / 256));
  // a ragged K needs a per-lane test only for a row-major operand
  if (p.K % kBK == 0 || (TA && TB))
    hipLaunchKernelGGL((k_gemm_pingpong<FA, FB, OUT, false, RW, BM, TR, TA, TB>), dim3(nb), dim3(512), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((k_gemm_pingpong<FA, FB, OUT, true, RW, BM, TR, TA, TB>), dim3(nb), dim3(512), 0,
                       stream, p);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus();

// Rounds of a grid of BM x 256 tiles over the CUs (one workgroup per CU at a
// time), weighted by the tile's rows: the cost model that picks the tile
// height.
inline int64_t tile_rounds_cost(int64_t M, int64_t N, int bm, int cus) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + 255) / 256);
  return ((tiles + cus - 1) / cus) * bm;
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool RW, bool TA = false, bool TB = false>
static hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  auto kern = k_gemm<BM, BN, WM, WN, FA, FB, OUT, RW, TA, TB>;
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

// The large-tile kernel addresses each operand through a buffer descriptor
// with 32-bit offsets: a row-major operand's 256-row panel, or a
// contraction-major operand's whole K rows (its per-lane "outside" offset is
// just below 2^31).
template <bool TA, bool TB>
inline bool big_tiles_fit(const GemmProblem& p) {
  const int64_t lim = (1ll << 31) - 256;
  return p.K > 0 && (TA ? p.K * p.M < lim : p.K * 256 < lim) && (TB ? p.K * p.N < lim : p.K * 256 < lim);
}

// The large-tile kernel's tiling of an M x N output on `cus` CUs: 256 x 256
// tiles, 224-row tiles along M, or (swap_ok) 224-row tiles along N with the
// operands' roles swapped, where their rounds over the CUs take clearly
// (5%) less time.  cus <= 0 (unknown) keeps 256 x 256.
enum BigTiling { kTile256, kTile224, kTile224Swapped };
inline BigTiling big_tiling(int64_t M, int64_t N, int cus, bool swap_ok) {
  if (cus <= 0) return kTile256;
  const int64_t c256 = tile_rounds_cost(M, N, 256, cus);
  const int64_t c224 = tile_rounds_cost(M, N, 224, cus);
  if (swap_ok && tile_rounds_cost(N, M, 224, cus) * 100 < (c224 < c256 ? c224 : c256) * 95)
    return kTile224Swapped;
  return c224 * 100 < c256 * 95 ? kTile224 : kTile256;
}
// Enough 256 x 256 tiles to fill the chip: the large-tile kernel's range.
inline bool big_tiles_wanted(int64_t M, int64_t N) {
  return ((M + 255) / 256) * ((N + 255) / 256) >= 128;
}

template <int FA, int FB, int OUT, bool RW, bool TA = false, bool TB = false>
static hipError_t launch_tiles(const GemmProblem& p, hipStream_t stream) {
  // The large-tile kernel in the tiling big_tiling picks.  The roles are not
  // swapped under row-wise scaling, nor where that would move a
  // contraction-major B into the A slot, whose fragments take twice the
  // transposed LDS reads of B's.
  if (big_tiles_wanted(p.M, p.N) && big_tiles_fit<TA, TB>(p)) {
    const BigTiling t = big_tiling(p.M, p.N, device_cus(), !RW && (TA || !TB));
    if constexpr (!RW && (TA || !TB)) {
      if (t == kTile224Swapped) {
        GemmProblem q = p;
        q.A = p.B;
        q.B = p.A;
        q.inv_a = p.inv_b;
        q.inv_b = p.inv_a;
        q.M = p.N;
        q.N = p.M;
        return launch_pingpong<FB, FA, OUT, RW, 224, true, TB, TA>(q, stream);
      }
    }
    if (t == kTile224) return launch_pingpong<FA, FB, OUT, RW, 224, false, TA, TB>(p, stream);
    return launch_pingpong<FA, FB, OUT, RW, 256, false, TA, TB>(p, stream);
  }
  return launch_cfg<128, 128, 2, 2, FA, FB, OUT, RW, TA, TB>(p, stream);
}

// Two problems: one launch of the 128 x 128 kernel when both take it,
// otherwise one launch each.
template <int FA, int FB, int OUT, bool RW, bool TA0 = false, bool TB0 = false, bool TA1 = false,
          bool TB1 = false>
static hipError_t launch_tiles_pair(const GemmProblem& p0, const GemmProblem& p1, hipStream_t stream) {
  auto big0 = ((p0.M + 255) / 256) * ((p0.N + 255) / 256) >= 128 && big_tiles_fit<TA0, TB0>(p0);
  auto big1 = ((p1.M + 255) / 256) * ((p1.N + 255) / 256) >= 128 && big_tiles_fit<TA1, TB1>(p1);
  if (big0 || big1) {
    hipError_t e = p0.M && p0.N ? launch_tiles<FA, FB, OUT, RW, TA0, TB0>(p0, stream) : hipSuccess;
    if (e != hipSuccess) return e;
    return p1.M && p1.N ? launch_tiles<FA, FB, OUT, RW, TA1, TB1>(p1, stream) : hipSuccess;
  }
  using Cfg = GemmCfg<128, 128, 2, 2>;
  auto kern = k_gemm2<128, 128, 2, 2, FA, FB, OUT, RW, TA0, TB0, TA1, TB1>;
  static bool attr_set = false;
  if (!attr_set && Cfg::kLdsBytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  const int64_t gx = cdiv(p0.N, 128) > cdiv(p1.N, 128) ? cdiv(p0.N, 128) : cdiv(p1.N, 128);
  const int64_t gy = cdiv(p0.M, 128) > cdiv(p1.M, 128) ? cdiv(p0.M, 128) : cdiv(p1.M, 128);
  if (gx == 0 || gy == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)gy, 2), dim3(Cfg::kThreads), Cfg::kLdsBytes,
                     stream, p0, p1);
  return hipGetLastError();
}

template <int FA, int FB, bool RW, bool TA = false, bool TB = false>
static hipError_t launch_out(const GemmProblem& p, int out, hipStream_t stream) {
  switch (out) {
    case FP8SG_OUT_BF16: return launch_tiles<FA, FB, FP8SG_OUT_BF16, RW, TA, TB>(p, stream);
    case FP8SG_OUT_F16: return launch_tiles<FA, FB, FP8SG_OUT_F16, RW, TA, TB>(p, stream);
    default: return launch_tiles<FA, FB, FP8SG_OUT_F32, RW, TA, TB>(p, stream);
  }
}

template <bool RW, bool TA = false, bool TB = false>
static hipError_t launch_gemm_any(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E4M3FN) return launch_out<0, 0, RW, TA, TB>(p, out, stream);
  if (fa == FP8SG_E5M2 && fb == FP8SG_E4M3FN) return launch_out<1, 0, RW, TA, TB>(p, out, stream);
  if (fa == FP8SG_E4M3FN && fb == FP8SG_E5M2) return launch_out<0, 1, RW, TA, TB>(p, out, stream);
  return launch_out<1, 1, RW, TA, TB>(p, out, stream);
}

}  // namespace fp8sg
