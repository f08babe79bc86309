// Scale + quantize-cast of bf16 (or fp16) tensors to OCP FP8, fused with the transposed
// copy [FP8-TRAIN §2: scale = fp8_max / amax in fp64, x * scale, clamp, cast;
// §3: e4m3 for activations and weights, e5m2 for gradients; §4: the backward
// GEMMs need each operand contiguous along its contraction dimension, which
// for x, W and gy means a transposed FP8 copy].
//
// Every block reduces the amax kernel's partial maxima (all 1024 slots, 4 KB,
// loaded together with its first tile) and recomputes the scale (two fp64
// divisions), so the amax -> scale step needs no launch of its own; the first
// block of each job also writes the record's amax and scale fields.
//
// Tiled path: one 128 x 128 tile per 256-thread block (blocks stride over the
// tiles when there are more tiles than blocks).  The tile is read once with
// 16-byte loads (8 in flight per thread), quantized in registers, stored
// row-major with coalesced 8-byte stores, staged in LDS (16 KB, XOR-swizzled
// so both the row-wise writes and the column-wise reads spread over the
// banks), transposed in 4x4-byte blocks with byte permutes, and stored to qT
// with 16-byte stores, 8 lanes per 128-byte row segment.  Tiles are walked in
// groups of 2 row tiles (tile_grouped): the blocks in flight together cover a
// short, wide band of the tensor.  HBM traffic is the algorithmic 2 B read +
// 1 B + 1 B written per element.
//
// Delayed scaling [PT-CH20 §20.5.9: each FP8 op keeps an amax history of its
// input; the scale comes from the amax of earlier steps]: with a history the
// blocks take the scale from the history's largest entry instead of the amax
// kernel's partials, and each block also reduces |x| over what it loaded and
// stores the result in its own partial slot of the record (at most
// FP8SG_AMAX_PARTS blocks per tensor; the tiled blocks then loop over tiles).
// k_hist_push then reduces those partials into rec->amax and pushes it to the
// front of the history.  One pass over x instead of two.  A tensor that needs
// more blocks than there are slots (more than 16 Mi elements) takes the
// two-level form: k_parts_clear zeroes the slots first, the cast runs one
// pass per block like the dynamic cast, and block b folds its maximum into
// slot b % FP8SG_AMAX_PARTS with an unsigned atomic max (the fp32 bits of
// non-negative values order like the values, NaN canonical above +inf; a
// maximum does not depend on the order of the updates).
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kQThreads = 256;
constexpr int kQTile = 128;

__device__ __forceinline__ const QuantJob& pick_job(const QuantArgs& a, int& lb) {
  int j = 0;
#pragma unroll
  for (int t = 1; t < kMaxQuantJobs; ++t)
    if (t < a.njobs && (int)blockIdx.x >= a.job[t].block0) j = t;
  lb = (int)blockIdx.x - a.job[j].block0;
  return a.job[j];
}

__device__ __forceinline__ void write_scale_fields(fp8sg_scale_rec* rec, float amax,
                                                   const ScaleVals& v) {
  rec->amax = amax;
  rec->scale = v.s;
  rec->inv = v.inv;
  rec->scale32 = v.s32;
  rec->inv32 = v.inv32;
}

// Where a job's scale comes from: the amax kernel's partials in its record,
// the largest entry of its amax history (delayed scaling), or an amax the
// caller supplies in device memory (taken as one history entry: NaN stays
// NaN, a negative value counts as 0).
enum ScaleSrc { kSrcParts = 0, kSrcHist = 1, kSrcGiven = 2 };
// The scale source's loads, issued ahead of the first tile's loads.
template <int SRC>
__device__ __forceinline__ const float* src_entries(const QuantJob& job, int32_t& n) {
  n = SRC == kSrcHist ? job.hist_len : 1;
  return SRC == kSrcHist ? job.hist : job.amax_in;
}

// The scale of a job: from the amax kernel's partials, the history or the
// caller's amax.
template <int SRC>
__device__ __forceinline__ float job_amax(const QuantJob& job) {
  if constexpr (SRC == kSrcHist) return hist_amax<kQThreads>(job.hist, job.hist_len);
  else if constexpr (SRC == kSrcGiven) return hist_amax<kQThreads>(job.amax_in, 1);
  else return amax_from_partials<kQThreads>(job.rec);
}

// SELF (a small tensor cast by one block): the block reduces |x| over the
// whole tensor itself, then casts it [FP8-TRAIN §2]; x is read twice, the
// second time from L2.  The amax also goes to the record's first partial
// slot, as if one amax block had written it.
__device__ __forceinline__ float self_amax(const QuantJob& job) {
  const int64_t nv = job.rows * job.cols / 8;  // cols % 16 == 0 on this path
  const uint4* xv = reinterpret_cast<const uint4*>(job.x);
  uint32_t m = 0;
  // eight loads in flight per thread (one at a time made a 32 Ki-element
  // tensor 16 dependent round trips); past the end a lane rereads vector 0,
  // an element of x, which leaves the maximum unchanged
  constexpr int kU = 8;
  for (int64_t k0 = threadIdx.x; k0 < nv; k0 += (int64_t)kQThreads * kU) {
    uint4 t[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + (int64_t)u * kQThreads;
      t[u] = xv[k < nv ? k : 0];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) m = absmax8(m, t[u]);
  }
  const uint32_t bits = block_max_u32<kQThreads>(absmax_bits(m));
  if (threadIdx.x == 0) {
    job.rec->_part[0] = bits;
    job.rec->_nparts = 1;
  }
  return __uint_as_float(bits);
}

// DELAYED: this block's |x| maximum (packed pair max m) into its partial slot
// (ATOMIC: folded into slot lb % FP8SG_AMAX_PARTS, which k_parts_clear zeroed).
static_assert((FP8SG_AMAX_PARTS & (FP8SG_AMAX_PARTS - 1)) == 0, "slot index by mask");
template <bool DELAYED, bool ATOMIC = false>
__device__ __forceinline__ void store_block_amax(const QuantJob& job, int lb, uint32_t m) {
  if constexpr (DELAYED && ATOMIC) {
    const uint32_t bits = block_max_u32<kQThreads>(absmax_bits(m));
    if (threadIdx.x == 0) atomicMax(&job.rec->_part[lb & (FP8SG_AMAX_PARTS - 1)], bits);
  } else if constexpr (DELAYED) {
    const uint32_t bits = block_max_u32<kQThreads>(absmax_bits(m));
    if (threadIdx.x == 0) {
      job.rec->_part[lb] = bits;
      if (lb == 0) job.rec->_nparts = (uint32_t)job.nblocks;
    }
    // as the amax kernel: the slots past the block count read as zero
    if (lb == 0)
      for (int i = job.nblocks + (int)threadIdx.x; i < FP8SG_AMAX_PARTS; i += kQThreads)
        job.rec->_part[i] = 0;
  }
}

// DELAYED writes the scale fields only: rec->amax is the current tensor's,
// published by k_hist_push.
template <bool DELAYED>
__device__ __forceinline__ void publish_scale(fp8sg_scale_rec* rec, float amax, const ScaleVals& v) {
  if constexpr (DELAYED) {
    rec->scale = v.s;
    rec->inv = v.inv;
    rec->scale32 = v.s32;
    rec->inv32 = v.inv32;
  } else {
    write_scale_fields(rec, amax, v);
  }
}

template <int FMT, bool S, int SRC, bool SELF = false, bool F16 = false, bool ATOMIC = false>
__global__ __launch_bounds__(kQThreads) void k_quant_tiled(QuantArgs args) {
  static_assert(!F16 || (SRC == kSrcParts && !SELF), "fp16 inputs: dynamic casts only");
  constexpr bool DELAYED = SRC == kSrcHist;
  constexpr bool kParts = SRC == kSrcParts && !SELF;  // scale from the amax kernel's partials
  int lb;
  const QuantJob& job = pick_job(args, lb);
  const int tid = threadIdx.x;
  const int64_t rows = job.rows, cols = job.cols;
  const int64_t tiles_r = (rows + kQTile - 1) / kQTile;
  const int64_t ntiles = tiles_r * job.tiles_c;
  __shared__ uint32_t lds[kQTile * 32];
  uint32_t am = 0;  // DELAYED: packed |x| max of everything this block loaded

  // phase 1 layout: 16 lanes per row (8 elements each), 16 rows per pass, 8 passes
  const int c8 = tid & 15;
  const int r0 = tid >> 4;
  uint4 v[8];
  // The one block of an empty tensor has no tile: it loads from its record
  // (valid memory, nothing stored), so that no branch precedes the first
  // loads.  A branch there makes the wait for the partials wait for the
  // tile's loads too (the wait count is taken from the path without them).
  const int64_t t0 = S ? xcd_contiguous(lb, job.nblocks) : lb;  // this block's first tile
  const bool has_tile = t0 < ntiles;
  const uint16_t* const x = has_tile ? job.x : reinterpret_cast<const uint16_t*>(job.rec);
  const int64_t tr_any = tiles_r > 0 ? tiles_r : 1;
  auto load = [&](int64_t tile) {
    int64_t rt, ct;
    tile_grouped(tile, tr_any, job.tiles_c, rt, ct);
    const int64_t gc = ct * kQTile + 8 * c8;
    const bool col_ok = gc < cols;  // cols % 16 == 0: a group of 8 is all in or all out
    // Every load is issued, with no branch between them: a lane outside a
    // ragged tile loads the tensor's first 8 elements instead.  Those codes
    // are never stored (rows and cols are multiples of 16, so each 8-column
    // group and each 16-row group of qT is all in or all out), and a delayed
    // amax over them is unchanged (they are elements of x).
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t gr = rt * kQTile + r0 + 16 * p;
      v[p] = ld16<S>(x + ((col_ok && gr < rows) ? gr * cols + gc : 0));
    }
  };
  // partials (or the history), then the first tile, all in flight before
  // the scale is derived
  float amax;
  if constexpr (kParts) {
    PartialLoads<kQThreads> parts;
    parts.issue(job.rec);
    load(has_tile ? t0 : 0);
    amax = parts.reduce();
  } else if constexpr (SRC != kSrcParts) {
    int32_t ne;
    const float* src = src_entries<SRC>(job, ne);
    HistLoads<kQThreads> hl;
    hl.issue(src, ne);
    load(has_tile ? t0 : 0);
    amax = hl.reduce();
  } else {
    amax = self_amax(job);
  }
  const ScaleVals sv = scale_from_amax(amax, FMT);
  if (lb == 0 && tid == 0) publish_scale<DELAYED>(job.rec, amax, sv);

  for (int64_t tile = t0; tile < ntiles; tile += job.nblocks) {
    int64_t rt, ct;
    tile_grouped(tile, tiles_r, job.tiles_c, rt, ct);
    const int64_t r_tile = rt * kQTile, c_tile = ct * kQTile;
    const int64_t gc = c_tile + 8 * c8;
    const bool col_ok = gc < cols;
    if (SELF || tile != t0) load(tile);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = r0 + 16 * p;
      const int64_t gr = r_tile + r;
      if constexpr (DELAYED) am = absmax8(am, v[p]);
      const uint2 c = quant8<FMT, F16>(v[p], sv.s32);
      if (col_ok && gr < rows) st8<S>(job.q + gr * cols + gc, c);
      *reinterpret_cast<uint2*>(&lds[r * 32 + ((2 * c8) ^ swz(r))]) = c;
    }
    __syncthreads();

    // phase 2: lane owns tile columns 4cq..4cq+3 and tile rows 16rq..16rq+15
    const int cq = tid >> 3;
    const int rq = tid & 7;
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
    const int64_t tr0 = r_tile + 16 * rq;
    const int64_t tc0 = c_tile + 4 * cq;
    if (tr0 < rows && tc0 < cols) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st16<S>(job.qT + (tc0 + j) * rows + tr0, make_uint4(o[j][0], o[j][1], o[j][2], o[j][3]));
    }
    if (tile + job.nblocks < ntiles) __syncthreads();  // the next tile reuses lds
  }
  store_block_amax<DELAYED, ATOMIC>(job, lb, am);
}

// Row-major codes only, any element count: grid-stride over 16-byte loads.
// Dynamic scaling and the two-level delayed form give every block one pass of
// kFlatUnroll loads per thread (up to kFlatMaxBlocks blocks; 2^28 elements at
// 6.5 TB/s against 6.1 with 4096 striding blocks); otherwise delayed scaling
// has at most FP8SG_AMAX_PARTS blocks, which stride with 8 loads in flight
// per thread.
template <int SRC, bool ATOMIC = false>
constexpr int flat_unroll() { return SRC == kSrcHist && !ATOMIC ? 8 : 4; }
constexpr int64_t kFlatMaxBlocks = 65536;

template <int FMT, bool S, int SRC, bool F16 = false, bool ATOMIC = false>
__global__ __launch_bounds__(kQThreads) void k_quant_flat(QuantArgs args) {
  static_assert(!F16 || SRC == kSrcParts, "fp16 inputs: dynamic casts only");
  constexpr bool DELAYED = SRC == kSrcHist;
  int lb;
  const QuantJob& job = pick_job(args, lb);
  const int tid = threadIdx.x;
  uint32_t am = 0;

  const int64_t n = job.rows * job.cols;
  const int64_t nvec = n >> 3;
  // an empty tensor's block loads from its record, as in the tiled kernel
  const uint4* const xv = reinterpret_cast<const uint4*>(
      nvec > 0 ? static_cast<const void*>(job.x) : static_cast<const void*>(job.rec));
  uint2* qv = reinterpret_cast<uint2*>(job.q);
  constexpr int kFlatUnroll = flat_unroll<SRC, ATOMIC>();
  const int64_t step = (int64_t)job.nblocks * kQThreads * kFlatUnroll;
  uint4 v[kFlatUnroll];
  // branch-free as in the tiled kernel: past the end a lane loads vector 0
  // (stored nowhere; an element of x, so a delayed amax is unchanged)
  auto load = [&](int64_t base) {
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
      const int64_t k = base + (int64_t)u * kQThreads;
      v[u] = ld16<S>(xv + (k < nvec ? k : 0));
    }
  };
  // as in the tiled kernel: partials, then the first loads, then the scale
  const int64_t base0 = (int64_t)lb * kQThreads * kFlatUnroll + tid;
  float amax;
  if constexpr (SRC == kSrcParts) {
    PartialLoads<kQThreads> parts;
    parts.issue(job.rec);
    load(base0);
    amax = parts.reduce();
  } else {
    int32_t ne;
    const float* src = src_entries<SRC>(job, ne);
    HistLoads<kQThreads> hl;
    hl.issue(src, ne);
    load(base0);
    amax = hl.reduce();
  }
  const ScaleVals sv = scale_from_amax(amax, FMT);
  if (lb == 0 && tid == 0) publish_scale<DELAYED>(job.rec, amax, sv);
  for (int64_t base = base0; base < nvec; base += step) {
    if (base != base0) load(base);
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
      const int64_t k = base + (int64_t)u * kQThreads;
      if constexpr (DELAYED) am = absmax8(am, v[u]);
      if (k < nvec) st8<S>(qv + k, quant8<FMT, F16>(v[u], sv.s32));
    }
  }
  if (lb == 0 && tid < (int)(n & 7)) {
    const int64_t i = (nvec << 3) + tid;
    if constexpr (DELAYED) am = pmax(am, (uint32_t)(job.x[i] & 0x7FFFu));
    job.q[i] = quant1<FMT, F16>(job.x[i], sv.s32);
  }
  store_block_amax<DELAYED, ATOMIC>(job, lb, am);
}

// Transposed copy of a shape the tiled kernel does not take: one thread per element.
template <int FMT, int SRC, bool F16 = false>
__global__ __launch_bounds__(kQThreads) void k_quant_elem(QuantArgs args) {
  static_assert(!F16 || SRC == kSrcParts, "fp16 inputs: dynamic casts only");
  constexpr bool DELAYED = SRC == kSrcHist;
  int lb;
  const QuantJob& job = pick_job(args, lb);
  const int tid = threadIdx.x;
  const float amax = job_amax<SRC>(job);
  const ScaleVals sv = scale_from_amax(amax, FMT);
  if (lb == 0 && tid == 0) publish_scale<DELAYED>(job.rec, amax, sv);
  uint32_t am = 0;
  const int64_t n = job.rows * job.cols;
  for (int64_t i = (int64_t)lb * kQThreads + tid; i < n; i += (int64_t)job.nblocks * kQThreads) {
    if constexpr (DELAYED) am = pmax(am, (uint32_t)(job.x[i] & 0x7FFFu));
    const uint8_t c = quant1<FMT, F16>(job.x[i], sv.s32);
    job.q[i] = c;
    const int64_t r = i / job.cols, cc = i - r * job.cols;
    job.qT[cc * job.rows + r] = c;
  }
  store_block_amax<DELAYED>(job, lb, am);
}

// Two-level delayed cast, before it: every partial slot of each job's record
// zeroed (the cast's blocks fold their maxima into them), all slots counted.
// One block per job.
__global__ __launch_bounds__(kQThreads) void k_parts_clear(QuantArgs args) {
  fp8sg_scale_rec* rec = args.job[blockIdx.x].rec;
  for (int i = threadIdx.x; i < FP8SG_AMAX_PARTS; i += kQThreads) rec->_part[i] = 0;
  if (threadIdx.x == 0) rec->_nparts = FP8SG_AMAX_PARTS;
}

// Delayed scaling, after the cast: rec->amax = the current tensor's amax
// (from the partials the cast left), pushed to the front of the history; the
// oldest entry drops out.  One block per job.
__global__ __launch_bounds__(kQThreads) void k_hist_push(QuantArgs args) {
  const QuantJob& job = args.job[blockIdx.x];
  // all partial slots and the history entries are loaded together (an index
  // past the history rereads entry 0; such values are never written back)
  PartialLoads<kQThreads> parts;
  parts.issue(job.rec);
  constexpr int kMaxPer = FP8SG_MAX_HISTORY / kQThreads;
  float old[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = threadIdx.x + k * kQThreads;
    old[k] = job.hist[i < job.hist_len ? i : 0];
  }
  const float a = parts.reduce();
  __syncthreads();  // every entry read before any is overwritten
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = threadIdx.x + k * kQThreads;
    if (i + 1 < job.hist_len) job.hist[i + 1] = old[k];
  }
  if (threadIdx.x == 0) {
    job.hist[0] = a;
    job.rec->amax = a;
  }
}

enum QuantPath { kPathTiled, kPathFlat, kPathElem };

static QuantPath path_of(const QuantJob& j) {
  if (!j.qT) return kPathFlat;
  if (j.rows % 16 == 0 && j.cols % 16 == 0) return kPathTiled;
  return kPathElem;
}

// Blocks of a job on path p.  atomic: the two-level delayed form (the block
// count is not bounded by the partial slots).
static int blocks_of(QuantJob& j, QuantPath p, bool atomic = false) {
  const int64_t n = j.rows * j.cols;
  int64_t b;
  if (p == kPathTiled) {
    const int64_t tr = (j.rows + kQTile - 1) / kQTile, tc = (j.cols + kQTile - 1) / kQTile;
    j.tiles_c = (int32_t)(tc > 0 ? tc : 1);
    b = tr * tc;
    if (b > (1 << 20)) b = 1 << 20;  // the blocks stride over the tiles
  } else if (p == kPathFlat) {
    const int64_t per = (int64_t)kQThreads *
        (j.hist ? (atomic ? flat_unroll<kSrcHist, true>() : flat_unroll<kSrcHist>()) : flat_unroll<kSrcParts>());
    b = ((n >> 3) + per - 1) / per;
    if (b > kFlatMaxBlocks) b = kFlatMaxBlocks;
  } else {
    b = (n + kQThreads - 1) / kQThreads;
    if (b > 4096) b = 4096;
  }
  if (j.hist && !atomic && b > FP8SG_AMAX_PARTS) b = FP8SG_AMAX_PARTS;  // one partial slot per block
  return (int)(b < 1 ? 1 : b);  // one block at least: it writes the scale fields
}

// Whether a delayed launch on path p takes the two-level form: some job
// needs more blocks for one pass than there are partial slots.
static bool two_level(const QuantArgs& a, int j0, int j1, QuantPath p) {
  if (p == kPathElem) return false;
  for (int j = j0; j < j1; ++j) {
    QuantJob jb = a.job[j];
    if (blocks_of(jb, p, true) > FP8SG_AMAX_PARTS) return true;
  }
  return false;
}

template <int FMT, int SRC, bool F16 = false>
static hipError_t launch_fmt(QuantArgs a, hipStream_t stream, bool self = false) {
  constexpr bool DELAYED = SRC == kSrcHist;
  // jobs of one launch must take the same path; otherwise split into launches
  for (int j0 = 0; j0 < a.njobs;) {
    const QuantPath p = path_of(a.job[j0]);
    QuantArgs sub{};
    int total = 0;
    int64_t bytes = 0;  // read + written by this launch
    int j = j0;
    while (j < a.njobs && path_of(a.job[j]) == p) ++j;
    const bool atomic = DELAYED && two_level(a, j0, j, p);
    for (int i = j0; i < j; ++i) {
      QuantJob jb = a.job[i];
      jb.nblocks = blocks_of(jb, p, atomic);
      if (self) jb.nblocks = 1;  // the block loops over all the tensor's tiles
      jb.block0 = total;
      total += jb.nblocks;
      bytes += jb.rows * jb.cols * (jb.qT ? 4 : 3);
      sub.job[sub.njobs++] = jb;
    }
    const bool st = bytes >= kStreamBytes;
    if constexpr (DELAYED) {
      if (atomic) {
        hipLaunchKernelGGL(k_parts_clear, dim3(sub.njobs), dim3(kQThreads), 0, stream, sub);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p == kPathTiled && st)
          hipLaunchKernelGGL((k_quant_tiled<FMT, true, SRC, false, false, true>), dim3(total), dim3(kQThreads), 0, stream, sub);
        else if (p == kPathTiled)
          hipLaunchKernelGGL((k_quant_tiled<FMT, false, SRC, false, false, true>), dim3(total), dim3(kQThreads), 0, stream, sub);
        else if (st)
          hipLaunchKernelGGL((k_quant_flat<FMT, true, SRC, false, true>), dim3(total), dim3(kQThreads), 0, stream, sub);
        else
          hipLaunchKernelGGL((k_quant_flat<FMT, false, SRC, false, true>), dim3(total), dim3(kQThreads), 0, stream, sub);
      }
    }
    if (atomic) {
      // launched above
    } else if (self && p == kPathTiled && SRC == kSrcParts && !F16)
      hipLaunchKernelGGL((k_quant_tiled<FMT, false, kSrcParts, true>), dim3(total), dim3(kQThreads), 0, stream, sub);
    else if (p == kPathTiled && st)
      hipLaunchKernelGGL((k_quant_tiled<FMT, true, SRC, false, F16>), dim3(total), dim3(kQThreads), 0, stream, sub);
    else if (p == kPathTiled)
      hipLaunchKernelGGL((k_quant_tiled<FMT, false, SRC, false, F16>), dim3(total), dim3(kQThreads), 0, stream, sub);
    else if (p == kPathFlat && st)
      hipLaunchKernelGGL((k_quant_flat<FMT, true, SRC, F16>), dim3(total), dim3(kQThreads), 0, stream, sub);
    else if (p == kPathFlat)
      hipLaunchKernelGGL((k_quant_flat<FMT, false, SRC, F16>), dim3(total), dim3(kQThreads), 0, stream, sub);
    else
      hipLaunchKernelGGL((k_quant_elem<FMT, SRC, F16>), dim3(total), dim3(kQThreads), 0, stream, sub);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (DELAYED) {
      hipLaunchKernelGGL(k_hist_push, dim3(sub.njobs), dim3(kQThreads), 0, stream, sub);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    j0 = j;
  }
  return hipSuccess;
}

bool self_cast_fits(const QuantArgs& a) {
  for (int j = 0; j < a.njobs; ++j) {
    const QuantJob& jb = a.job[j];
    if (jb.hist || path_of(jb) != kPathTiled || jb.rows * jb.cols > kSelfCastMaxElems) return false;
  }
  return a.njobs > 0;
}

hipError_t launch_quantize_self(QuantArgs args, int fmt, hipStream_t stream) {
  return fmt == FP8SG_E4M3FN ? launch_fmt<FP8SG_E4M3FN, kSrcParts>(args, stream, true)
                             : launch_fmt<FP8SG_E5M2, kSrcParts>(args, stream, true);
}

hipError_t launch_quantize(QuantArgs args, int fmt, hipStream_t stream) {
  // jobs with different scale sources are never mixed in one call (the entry
  // points build the job lists)
  const bool delayed = args.njobs > 0 && args.job[0].hist;
  const bool given = args.njobs > 0 && args.job[0].amax_in;
  if (args.in_f16)  // fp16 inputs: dynamic scaling from the amax kernel's partials
    return fmt == FP8SG_E4M3FN ? launch_fmt<FP8SG_E4M3FN, kSrcParts, true>(args, stream)
                               : launch_fmt<FP8SG_E5M2, kSrcParts, true>(args, stream);
  if (delayed)
    return fmt == FP8SG_E4M3FN ? launch_fmt<FP8SG_E4M3FN, kSrcHist>(args, stream)
                               : launch_fmt<FP8SG_E5M2, kSrcHist>(args, stream);
  if (given)
    return fmt == FP8SG_E4M3FN ? launch_fmt<FP8SG_E4M3FN, kSrcGiven>(args, stream)
                               : launch_fmt<FP8SG_E5M2, kSrcGiven>(args, stream);
  return fmt == FP8SG_E4M3FN ? launch_fmt<FP8SG_E4M3FN, kSrcParts>(args, stream)
                             : launch_fmt<FP8SG_E5M2, kSrcParts>(args, stream);
}

}  // namespace fp8sg
