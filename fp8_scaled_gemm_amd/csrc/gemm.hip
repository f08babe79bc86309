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

// ---------------------------------------------------------------------------
// Large-tile kernel: BM x BN x 128 tiles streamed global -> LDS by the buffer
// unit (buffer_load_dwordx4 ... lds), two LDS stages, so the next k-tile's
// loads are in flight while the current one is multiplied, with no VGPR
// staging.  One load instruction moves 64 lanes x 16 B = 1 KB = 8 rows of a
// 128-byte k-slice; lane l fills LDS row 8g + l/8, chunk l%8, and fetches the
// global chunk that belongs there under the swizzle.  The per-block buffer
// descriptor spans only the block's row panel, so rows past M (or N) read as
// zero; chunks past K are pointed outside the descriptor and read as zero too.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte chunk c of LDS row r lives at chunk c ^ swz16(r).  swz16 is a
// bijection on every aligned group of 8 rows and on the even and the odd rows
// of every aligned group of 16, so the 16-byte fragment reads hit distinct
// banks whether the LDS serves 8 lanes x 16 B or 16 lanes x 16 B per cycle.
__device__ __forceinline__ int swz16(int r) { return (r ^ (r >> 3)) & 7; }
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

#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Position of this block's tile.  Workgroups are handed to the 8 XCDs round
// robin (block b on XCD b % 8); renumber so that each XCD gets a run of
// consecutive tile indices, then walk tiles in groups of kGroupM tile-rows,
// column by column, so one XCD's tiles form a compact region whose A and B
// panels its L2 can share.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_of(int nbm, int nbn, int& tm, int& tn) {
  const int nb = nbm * nbn;
  const int b = blockIdx.x;
  const int q = nb / 8, rem = nb % 8, x = b % 8;
  const int t = x * q + (x < rem ? x : rem) + b / 8;
  const int per_group = kGroupM * nbn;
  const int g = t / per_group, r = t % per_group;
  const int gm = (nbm - g * kGroupM) < kGroupM ? (nbm - g * kGroupM) : kGroupM;
  tm = g * kGroupM + r % gm;
  tn = r / gm;
}

// The two pipeline stages are separate LDS objects and the k-loop is unrolled
// by two, so every fragment read names its stage at compile time: the
// compiler can then prove the reads do not alias the buffer loads still
// filling the other stage and waits only for the loads of the stage it reads.
template <int BM, int BN>
struct LdsStages {
  static constexpr int kA = BM * kBK, kB = BN * kBK;
};

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT>
__global__ __launch_bounds__(WM* WN* kWave) void k_gemm_lds(GemmProblem p) {
  constexpr int kNW = WM * WN;
  constexpr int kTM = BM / WM / 16, kTN = BN / WN / 16;
  constexpr int kIA = BM / 8 / kNW, kIB = BN / 8 / kNW;  // 1 KB loads per wave per k-tile
  static_assert(kIA * 8 * kNW == BM && kIB * 8 * kNW == BN, "tile rows / waves");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "16-row blocks");
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BN * kBK];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int nbm = (int)((M + BM - 1) / BM), nbn = (int)((N + BN - 1) / BN);
  int tm, tn;
  tile_of(nbm, nbn, tm, tn);
  const int64_t bm = (int64_t)tm * BM, bn = (int64_t)tn * BN;
  const int nk = (int)((K + kBK - 1) / kBK);

  const int64_t rows_a = (M - bm) < BM ? (M - bm) : BM;
  const int64_t rows_b = (N - bn) < BN ? (N - bn) : BN;
  const i32x4 ra = make_rsrc(p.A + bm * K, rows_a * K);
  const i32x4 rb = make_rsrc(p.B + bn * K, rows_b * K);

  // LDS row 8g + l/8, chunk l%8 of a k-tile holds global chunk (l%8) ^ swz16(row):
  // one load instruction moves 8 full 128-byte rows.
  auto chunk_of = [&](int g) { return (lane & 7) ^ swz16(8 * g + (lane >> 3)); };
  auto row_of = [&](int g) { return 8 * g + (lane >> 3); };
  auto issue = [&](int kt, uint8_t* a, uint8_t* b) {  // kt >= nk loads zeros
    const int k0 = kt < nk ? kt * kBK : (int)K;
#pragma unroll
    for (int i = 0; i < kIA; ++i) {
      const int g = wave * kIA + i, c = chunk_of(g);
      const uint32_t off = (k0 + 16 * c < K) ? (uint32_t)(row_of(g) * K + k0 + 16 * c) : kOob;
      lds_dma16(lds_addr(a + g * 1024), off, ra);
    }
#pragma unroll
    for (int i = 0; i < kIB; ++i) {
      const int g = wave * kIB + i, c = chunk_of(g);
      const uint32_t off = (k0 + 16 * c < K) ? (uint32_t)(row_of(g) * K + k0 + 16 * c) : kOob;
      lds_dma16(lds_addr(b + g * 1024), off, rb);
    }
  };

  v4f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // fragment of 16-row block rb: lane l holds row 16 rb + (l & 15), k bytes
  // [32 (l >> 4), +32) as two 16-byte chunks (the same k mapping for A and B)
  const int frow = lane & 15;
  const int fchunk = 2 * (lane >> 4);
  auto frag = [&](const uint8_t* base, int rb) {
    const int r = 16 * rb + frow;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + lds_off2(r, fchunk));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + lds_off2(r, fchunk + 1));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  const int ra0 = wm * (BM / WM) / 16;  // first 16-row block of this wave's A rows
  const int rb0 = wn * (BN / WN) / 16;

  // Fragments in registers: the kTN B fragments, two A fragments (the one
  // in use and the one being read), and one more A fragment at the tile
  // boundary.
  v8i bf[kTN];
  v8i af[2];
  auto mma1 = [&](int i, int j, const v8i& a_frag) {
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], a_frag, acc[i][j], FB,
                                                                 FA, 0, 0, 0, 0);
  };
  constexpr int kHold = 2;  // the last two A fragments x the last two B fragments wait
  static_assert(kTM >= kHold && kTN >= kHold && kTM % 2 == 0, "tile split");

  // One k-tile whose head fragments (A0, B*) are in registers or in flight.
  // A fragments are read one step ahead of their MFMAs.  The kHold x kHold
  // MFMAs that use the last A and the last B fragments are held back past the
  // barrier: once every wave has finished reading this stage and the next
  // tile has landed, each wave reads the next tile's A0 and first B
  // fragments into the registers already free, runs the held-back MFMAs
  // while those reads are in flight, then reads the remaining B fragments.
  // The matrix pipe therefore has work queued across the barrier.  Then the
  // freed stage is refilled with tile kt + 2.
  auto tile = [&](int kt, const uint8_t* a, const uint8_t* b, const uint8_t* na,
                  const uint8_t* nb, uint8_t* ra_next, uint8_t* rb_next) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      if (i + 1 < kTM) af[(i + 1) & 1] = frag(a, ra0 + i + 1);
      __builtin_amdgcn_sched_barrier(0);  // the read goes out before the MFMAs
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        if (i < kTM - kHold || j < kTN - kHold) mma1(i, j, af[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();                     // tile kt + 1 has landed (my part)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): all my reads of this stage returned
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    // branch-free: past the last tile these reads are stale and unused, and
    // the refill loads zeros
    const v8i na0 = frag(na, ra0);
#pragma unroll
    for (int j = 0; j < kTN - kHold; ++j) bf[j] = frag(nb, rb0 + j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = kTM - kHold; i < kTM; ++i)
#pragma unroll
      for (int j = kTN - kHold; j < kTN; ++j) mma1(i, j, af[i & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = kTN - kHold; j < kTN; ++j) bf[j] = frag(nb, rb0 + j);
    af[0] = na0;
    issue(kt + 2, ra_next, rb_next);
  };

  // Prologue: load tile 0; once it is in, load tile 1 and read tile 0's head
  // fragments.
  issue(0, sA0, sB0);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  af[0] = frag(sA0, ra0);
#pragma unroll
  for (int j = 0; j < kTN; ++j) bf[j] = frag(sB0, rb0 + j);
  issue(1, sA1, sB1);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    tile(kt, sA0, sB0, sA1, sB1, sA0, sB0);
    tile(kt + 1, sA1, sB1, sA0, sB0, sA1, sB1);
  }
  if (kt < nk) tile(kt, sA0, sB0, sA1, sB1, sA0, sB0);

  const float alpha = (float)(*p.inv_a * *p.inv_b);
  if constexpr (OUT == FP8SG_OUT_F32) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int64_t m = bm + wm * (BM / WM) + 16 * i + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int64_t n = bn + wn * (BN / WN) + 16 * j + 4 * (lane >> 4);
        if (n >= N) continue;
        v4f c = acc[i][j];
        c[0] *= alpha;
        c[1] *= alpha;
        c[2] *= alpha;
        c[3] *= alpha;
        store4<OUT>(p.C, m * N + n, c);
      }
    }
  } else {
    // 16-bit output: stage the BM x BN tile in the (now idle) LDS stages, then
    // write it out as whole row segments, 16 bytes per lane.  Row R of the
    // tile lives in stage array R / 64 (64 rows of 2 * BN bytes each); its
    // 16-byte chunk c sits at chunk c ^ (R & 31), so both the column-wise
    // writes of the accumulator layout and the row-wise reads spread over the
    // banks.
    static_assert(BM == 256 && BN == 256, "the staged epilogue assumes 256 x 256 tiles");
    constexpr int kRowBytes = 2 * BN;
    auto crow = [&](int r) -> uint8_t* {
      uint8_t* base = r < 64 ? sA0 : r < 128 ? sB0 : r < 192 ? sA1 : sB1;
      return base + (r & 63) * kRowBytes;
    };
    __builtin_amdgcn_s_waitcnt(0);  // no load may still be writing a stage
    __builtin_amdgcn_s_barrier();
    compiler_fence();
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int r = wm * (BM / WM) + 16 * i + (lane & 15);
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int col = wn * (BN / WN) + 16 * j + 4 * (lane >> 4);
        v4f c = acc[i][j];
        c[0] *= alpha;
        c[1] *= alpha;
        c[2] *= alpha;
        c[3] *= alpha;
        const int off = (((col >> 3) ^ (r & 31)) << 4) + (col & 7) * 2;
        store4<OUT>(crow(r) + off, 0, c);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    constexpr int kChunks = BN / 8;                       // 16-byte chunks per row
    constexpr int kRowsPerPass = kNW * kWave / kChunks;   // rows written per pass
    const int cc = threadIdx.x % kChunks;
#pragma unroll
    for (int pass = 0; pass < BM / kRowsPerPass; ++pass) {
      const int r = pass * kRowsPerPass + threadIdx.x / kChunks;
      const uint4 v = *reinterpret_cast<const uint4*>(crow(r) + ((cc ^ (r & 31)) << 4));
      const int64_t m = bm + r, n = bn + 8 * cc;
      if (m < M && n < N)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.C) + m * N + n) = v;
    }
  }
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT>
static hipError_t launch_lds(const GemmProblem& p, hipStream_t stream) {
  auto kern = k_gemm_lds<BM, BN, WM, WN, FA, FB, OUT>;
  const unsigned nb = (unsigned)(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN));
  hipLaunchKernelGGL(kern, dim3(nb), dim3(WM * WN * kWave), 0, stream, p);
  return hipGetLastError();
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
  // 256 x 256 tiles once there are enough of them to fill the chip
  const int64_t big = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  if (big >= 128 && p.K * 256 < (1ll << 31)) return launch_lds<256, 256, 2, 4, FA, FB, OUT>(p, stream);
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
