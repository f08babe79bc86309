// Device-side helpers shared by the fp8sg kernels (gfx950 / CDNA4).
//
// Sources (web pages; cited by title and section):
//   [FP8-TRAIN]  "FP8训练：量化、自动微分、Torchao" (lzwjava.github.io)
//   [PT-CH20]    "第20章 量化与混合精度训练" (yangyitao.com, PyTorch book ch. 20)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8sg.h"

namespace fp8sg {

constexpr int kWave = 64;

// Largest finite values of the two FP8 formats [FP8-TRAIN §2, §3 table].
constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;
// Lower clamp of amax in the scale division; the page names EPS without a value.
constexpr double kScaleEps = 1e-12;

// Streaming (non-temporal) 16- and 8-byte global accesses for data touched
// once per pass: the caches are told not to keep the lines, which lets a
// pure stream run at close to the HBM rate (measured on MI355X: reads 3.8 ->
// 6.7 TB/s, read + write 4.5 -> 6.3 TB/s for 512 MiB passes).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_stream(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}

// A pass that moves less than the Infinity Cache (256 MB) keeps ordinary
// cached accesses: its inputs were usually just written or read by the
// previous kernel and are still there, and its outputs are read next.
constexpr int64_t kStreamBytes = 256ll << 20;
// A GEMM output of this size or more leaves the kernel with non-temporal
// stores.  The GEMM is bound by its matrix cores and reads its operands at a
// small fraction of the memory bandwidth, so its output reaches HBM during
// the GEMM; stored cached, it would stay in the caches as dirty lines that
// the next memory-bound kernel, reading other tensors, has to write back
// first.  A smaller output stays cached for the consumer that reads it next.
constexpr int64_t kStreamOutBytes = 64ll << 20;
// An empty use of a loaded value (no instruction): the compiler may not sink
// the load into a later conditional use, where it would be issued only after
// the work before that use.
__device__ __forceinline__ void keep_loaded(const uint4& v) {
  asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

template <bool S>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (S) return ld_stream(p);
  else return *reinterpret_cast<const uint4*>(p);
}
template <bool S>
__device__ __forceinline__ void st16(void* p, uint4 v) {
  if constexpr (S) st_stream(p, v);
  else *reinterpret_cast<uint4*>(p) = v;
}
template <bool S>
__device__ __forceinline__ void st8(void* p, uint2 v) {
  if constexpr (S) st_stream(p, v);
  else *reinterpret_cast<uint2*>(p) = v;
}

__device__ __forceinline__ float fmt_max(int fmt) { return fmt == FP8SG_E4M3FN ? kE4M3Max : kE5M2Max; }

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-tensor scale from the amax word [FP8-TRAIN §2]: s = fp8_max / max(amax, EPS)
// as an IEEE fp64 division (NaN amax keeps NaN), inverse = 1/s in fp64, both also
// rounded to fp32.
struct ScaleVals {
  double s, inv;
  float s32, inv32;
};

__device__ __forceinline__ ScaleVals scale_from_amax(float amax, int fmt) {
  ScaleVals v;
  double d = (double)amax;
  if (d != d) {
    v.s = d;
  } else {
    if (d < kScaleEps) d = kScaleEps;
    v.s = (double)fmt_max(fmt) / d;
  }
  v.inv = 1.0 / v.s;
  v.s32 = (float)v.s;
  v.inv32 = (float)v.inv;
  return v;
}

// Keeps x as an fp32 value: an fp16 conversion that follows rounds this fp32
// value (two roundings, as the definition fl32 then fp16 has it), instead of
// being folded with the multiply that produced x into one mixed-precision
// instruction (v_fma_mixlo_f16) that rounds the exact product once.
__device__ __forceinline__ float fp32_value(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 fp32_value(f32x2 x) {
  asm volatile("" : "+v"(x));
  return x;
}

// clamp(y, -max, max) that keeps NaN (v_min/v_max return the non-NaN operand).
__device__ __forceinline__ float clamp_keep_nan(float y, float m) {
  float c = fminf(fmaxf(y, -m), m);
  return (y != y) ? y : c;
}

// Four already-clamped fp32 values -> four FP8 codes (byte i = value i), using
// gfx950's OCP converts, which round to nearest even.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r;
  if constexpr (FMT == FP8SG_E4M3FN) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  }
  return (uint32_t)r;
}

// The 16-bit input of a cast as fp32 (exact): bf16, the layer's dtype, or
// fp16 (F16: an fp16 model under loss scaling).  lo/hi: the element in the
// low / high half of a dword.
template <bool F16>
__device__ __forceinline__ float in_lo(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  else return bf16_lo(w);
}
template <bool F16>
__device__ __forceinline__ float in_hi(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else return bf16_hi(w);
}

// Quantize 8 inputs (one 16-byte load) to 8 codes (two dwords)
// [FP8-TRAIN §2: fl32(x * scale32), clamp, cast].
template <int FMT, bool F16 = false>
__device__ __forceinline__ uint2 quant8(uint4 v, float s32) {
  constexpr float m = FMT == FP8SG_E4M3FN ? kE4M3Max : kE5M2Max;
  float f0 = clamp_keep_nan(in_lo<F16>(v.x) * s32, m), f1 = clamp_keep_nan(in_hi<F16>(v.x) * s32, m);
  float f2 = clamp_keep_nan(in_lo<F16>(v.y) * s32, m), f3 = clamp_keep_nan(in_hi<F16>(v.y) * s32, m);
  float f4 = clamp_keep_nan(in_lo<F16>(v.z) * s32, m), f5 = clamp_keep_nan(in_hi<F16>(v.z) * s32, m);
  float f6 = clamp_keep_nan(in_lo<F16>(v.w) * s32, m), f7 = clamp_keep_nan(in_hi<F16>(v.w) * s32, m);
  return make_uint2(cvt4<FMT>(f0, f1, f2, f3), cvt4<FMT>(f4, f5, f6, f7));
}

template <int FMT, bool F16 = false>
__device__ __forceinline__ uint8_t quant1(uint16_t b, float s32) {
  constexpr float m = FMT == FP8SG_E4M3FN ? kE4M3Max : kE5M2Max;
  float f = clamp_keep_nan(in_lo<F16>(b) * s32, m);
  return (uint8_t)(cvt4<FMT>(f, 0.f, 0.f, 0.f) & 0xFFu);
}

// Maximum over the 16 lanes of a DPP row (lanes 16k .. 16k + 15), in every lane
// of the row: pairs (quad_perm 1,0,3,2), quads (2,3,0,1), half rows
// (row_half_mirror), rows (row_mirror).  All 64 lanes must be active.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  auto mx = [](uint32_t a, int b) { return (uint32_t)b > a ? (uint32_t)b : a; };
  v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Block-wide max of one u32 per thread; every thread gets the result.
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[NT / kWave];
  v = wave_max_u32(v);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = red[w] > r ? red[w] : r;
  __syncthreads();  // the next call may reuse red[]
  return r;
}

// amax of a tensor from the per-block partial maxima the amax kernel left in
// its record (fp32 bit patterns of non-negative values, NaN already
// canonical, so integer max is numeric max).  Called once per block by every
// thread; every thread gets the result.
template <int NT>
__device__ __forceinline__ float amax_from_partials(const fp8sg_scale_rec* rec) {
  const uint32_t np = rec->_nparts;
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < np; i += NT) {
    const uint32_t v = rec->_part[i];
    m = v > m ? v : m;
  }
  return __uint_as_float(block_max_u32<NT>(m));
}

// The same maximum as a cast block takes it: all FP8SG_AMAX_PARTS slots (the
// amax kernel zeroes the slots past its block count; zero never raises the
// maximum), a fixed number of loads per thread that depend on no other load.
// A block issues them before its data loads and then waits for them alone
// (the vector memory counter retires loads in order), so the partials' round
// trip overlaps the data's instead of preceding it.
template <int NT>
struct PartialLoads {
  static constexpr int kPer = FP8SG_AMAX_PARTS / NT;
  static_assert(FP8SG_AMAX_PARTS % NT == 0, "slots split evenly over the threads");
  uint32_t v[kPer];
  __device__ __forceinline__ void issue(const fp8sg_scale_rec* rec) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = rec->_part[threadIdx.x + k * NT];
  }
  __device__ __forceinline__ float reduce() const {
    uint32_t m = v[0];
#pragma unroll
    for (int k = 1; k < kPer; ++k) m = v[k] > m ? v[k] : m;
    return __uint_as_float(block_max_u32<NT>(m));
  }
};

// |x| max over bf16 pairs: packed 16-bit max of the bit patterns with the sign
// cleared (integer order = numeric order for non-negative IEEE values, every
// NaN above +inf).
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pmax(uint32_t a, uint32_t b) {
  us2 r = __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b));
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t absmax8(uint32_t m, uint4 v) {
  constexpr uint32_t mask = 0x7FFF7FFFu;
  m = pmax(m, v.x & mask);
  m = pmax(m, v.y & mask);
  m = pmax(m, v.z & mask);
  return pmax(m, v.w & mask);
}
// packed pair max -> fp32 bits of the larger magnitude, NaN made canonical
template <bool F16 = false>
__device__ __forceinline__ uint32_t absmax_bits(uint32_t m) {
  const uint32_t code = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
  if constexpr (F16) {  // fp16 magnitude: exact in fp32; inf stays inf
    if (code > 0x7C00u) return 0x7FC00000u;
    return __float_as_uint((float)__builtin_bit_cast(_Float16, (uint16_t)code));
  } else {
    const uint32_t bits = code << 16;
    return bits > 0x7F800000u ? 0x7FC00000u : bits;
  }
}

// Largest entry of an amax history (fp32, most recent first): NaN if any
// entry is NaN; negative entries count as 0.  Every thread gets the result.
template <int NT>
__device__ __forceinline__ float hist_amax(const float* hist, int32_t h) {
  uint32_t m = 0;
  for (int32_t i = threadIdx.x; i < h; i += NT) {
    uint32_t b = __float_as_uint(hist[i]);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) b = 0x7FC00000u;
    else if (b >> 31) b = 0;
    m = b > m ? b : m;
  }
  return __uint_as_float(block_max_u32<NT>(m));
}

// The same maximum with loads a block can issue ahead of its data loads (as
// PartialLoads): FP8SG_MAX_HISTORY / NT per thread, an index past the history
// reading entry 0 again (h >= 1), which cannot change the maximum.
template <int NT>
struct HistLoads {
  static constexpr int kPer = FP8SG_MAX_HISTORY / NT;
  static_assert(FP8SG_MAX_HISTORY % NT == 0, "entries split evenly over the threads");
  uint32_t v[kPer];
  __device__ __forceinline__ void issue(const float* hist, int32_t h) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int32_t i = (int32_t)threadIdx.x + k * NT;
      v[k] = __float_as_uint(hist[i < h ? i : 0]);
    }
  }
  __device__ __forceinline__ float reduce() const {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      uint32_t b = v[k];
      if ((b & 0x7FFFFFFFu) > 0x7F800000u) b = 0x7FC00000u;
      else if (b >> 31) b = 0;
      m = b > m ? b : m;
    }
    return __uint_as_float(block_max_u32<NT>(m));
  }
};

// Transposed stores of 128 x 128 code tiles (quantize.hip, rowwise.hip).
// Tile t of a tiles_r x tiles_c grid, walked in groups of 2 row tiles: down
// the 2 rows of a group first, then across its columns.  The blocks in flight
// together then cover a short, wide band: their row-major stores and loads
// form long runs in each row, and their transposed stores land in pairs of
// adjacent 128-byte pieces.  Measured at HBM scale against groups of 1, 4, 8,
// 16 and 32 rows and a diagonal and a hashed walk, 2 rows was fastest or
// near it on every shape (16384^2: 206 -> 199 us; 8192 x 14336: 96 -> 89 us;
// 8192 x 28672: 197 -> 178 us against 8-row groups).
// In 32-bit arithmetic (64-bit division is a long software loop): with rows,
// cols <= FP8SG_MAX_DIM and rows * cols <= FP8SG_MAX_ELEMS there are fewer
// than 2^24 tiles and 8 * tiles_c < 2^26.
__host__ __device__ inline void tile_grouped(int64_t t, int64_t tiles_r, int64_t tiles_c,
                                             int64_t& rt, int64_t& ct) {
  constexpr uint32_t G = 2;
  const uint32_t t32 = (uint32_t)t, tr = (uint32_t)tiles_r;
  const uint32_t per = G * (uint32_t)tiles_c, g = t32 / per, first = g * G;
  const uint32_t gs = tr - first < G ? tr - first : G;
  const uint32_t w = t32 - g * per;
  rt = first + w % gs;
  ct = w / gs;
}
static_assert((FP8SG_MAX_ELEMS >> 14) + 2 * (FP8SG_MAX_DIM >> 7) + 1 < (1ll << 24),
              "tile counts fit 32-bit arithmetic");

// Block -> first tile of a cast that streams from HBM: block b runs on XCD
// b % 8 (round-robin dispatch), and each XCD takes a contiguous eighth of the
// n first tiles, so the transposed stores of tiles that are neighbours in
// tile_grouped order leave through the same L2 (16384^2 with transposed copy:
// 218 -> 205 us; cached sizes gain nothing).  A bijection on [0, n).
__device__ __forceinline__ int64_t xcd_contiguous(int64_t b, int64_t n) {
  const int64_t q = n / 8, rem = n % 8, x = b % 8;
  return x * q + (x < rem ? x : rem) + b / 8;
}

// LDS tile: 128 rows x 32 dwords; dword column x of row r lives at x ^ swz(r).
__device__ __forceinline__ int swz(int r) { return ((r >> 4) & 3) << 3; }

// 4x4 byte transpose: out[j] byte i = in[i] byte j.
__device__ __forceinline__ void tr4x4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                      uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  // v_perm_b32(hi, lo, sel): selector bytes 0-3 pick lo's bytes, 4-7 hi's bytes
  uint32_t e0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);  // d0.b0 d1.b0 d0.b1 d1.b1
  uint32_t e1 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);  // d0.b2 d1.b2 d0.b3 d1.b3
  uint32_t f0 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
  uint32_t f1 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
  o0 = __builtin_amdgcn_perm(f0, e0, 0x05040100u);  // d0.b0 d1.b0 d2.b0 d3.b0
  o1 = __builtin_amdgcn_perm(f0, e0, 0x07060302u);  // d0.b1 d1.b1 d2.b1 d3.b1
  o2 = __builtin_amdgcn_perm(f1, e1, 0x05040100u);
  o3 = __builtin_amdgcn_perm(f1, e1, 0x07060302u);
}

}  // namespace fp8sg
