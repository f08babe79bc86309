// amax = max_i |x_i| over bf16 (or fp16) tensors [FP8-TRAIN §2: x.float().abs().max()].
//
// One pass over HBM, 2 bytes per element.  |x| is compared as the unsigned
// integer bits & 0x7FFF: for non-negative IEEE values (inf and NaN included)
// integer order is numeric order, so the maximum is exact, order-free and
// NaN-propagating (every NaN pattern sits above +inf).  Two bf16 lanes per
// dword are reduced together with packed 16-bit max.
//
// Stages: per-thread grid-stride loop over 16-byte loads (8 in flight) ->
// wavefront shuffle -> LDS across the block's waves -> one plain store of the
// block's maximum into its own slot of the record (at most FP8SG_AMAX_PARTS
// blocks; the first block zeroes the slots past the block count).  No atomics
// and no fences: same-address device-scope atomics from thousands of blocks
// serialise at one memory channel, which made an atomic-max design several
// times slower than the loads.  The consumer reduces the slots: every block
// of the quantize kernel loads all of them (4 KB) together with its first
// tile, and the standalone entry point adds a one-block finalize.
//
// Several tensors can share one launch (the forward pass reduces x and W
// together): each job owns a contiguous range of blocks.
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxUnroll = 8;  // 16-byte loads in flight per thread per iteration

template <bool S, bool F16 = false>
__global__ __launch_bounds__(kAmaxThreads) void k_amax(AmaxArgs args) {
  int j = 0;
#pragma unroll
  for (int t = 1; t < kMaxAmaxJobs; ++t)
    if (t < args.njobs && (int)blockIdx.x >= args.job[t].block0) j = t;
  const AmaxJob& job = args.job[j];
  const int lb = (int)blockIdx.x - job.block0;
  const int tid = threadIdx.x;

  const uint4* xv = reinterpret_cast<const uint4*>(job.x);
  const int64_t nvec = job.n >> 3;
  const int64_t step = (int64_t)job.nblocks * kAmaxThreads * kAmaxUnroll;
  const uint32_t mask = 0x7FFF7FFFu;
  uint32_t m = 0;
  for (int64_t base = (int64_t)lb * kAmaxThreads * kAmaxUnroll + tid; base < nvec; base += step) {
    uint4 v[kAmaxUnroll];
    // branch-free: past the end a lane loads vector 0 again, an element of x
    // (inside this loop nvec > 0), which leaves the maximum unchanged
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t k = base + (int64_t)u * kAmaxThreads;
      v[u] = ld16<S>(xv + (k < nvec ? k : 0));
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      m = pmax(m, v[u].x & mask);
      m = pmax(m, v[u].y & mask);
      m = pmax(m, v[u].z & mask);
      m = pmax(m, v[u].w & mask);
    }
  }
  // elements past the last full 16-byte vector
  if (lb == 0 && tid < (int)(job.n & 7)) m = pmax(m, (uint32_t)(job.x[(nvec << 3) + tid] & 0x7FFFu));

  // the largest magnitude as fp32 bits, any NaN canonical
  const uint32_t bits = block_max_u32<kAmaxThreads>(absmax_bits<F16>(m));
  if (tid == 0) {
    job.rec->_part[lb] = bits;
    if (lb == 0) job.rec->_nparts = (uint32_t)job.nblocks;
  }
  // the slots past the block count read as zero, so a consumer may take all
  // of them without reading the count first
  if (lb == 0)
    for (int i = job.nblocks + tid; i < FP8SG_AMAX_PARTS; i += kAmaxThreads) job.rec->_part[i] = 0;
}

// Standalone amax: publish rec->amax from the partial maxima (one block per job).
__global__ __launch_bounds__(kAmaxThreads) void k_amax_finalize(AmaxArgs args) {
  fp8sg_scale_rec* rec = args.job[blockIdx.x].rec;
  PartialLoads<kAmaxThreads> parts;  // every slot at once (unused ones are zero)
  parts.issue(rec);
  const float a = parts.reduce();
  if (threadIdx.x == 0) rec->amax = a;
}

int amax_blocks_for(int64_t n) {
  const int64_t nvec = n >> 3;
  const int64_t per_block = (int64_t)kAmaxThreads * kAmaxUnroll;
  int64_t b = (nvec + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > FP8SG_AMAX_PARTS) b = FP8SG_AMAX_PARTS;
  return (int)b;
}

hipError_t launch_amax(AmaxArgs args, bool finalize, hipStream_t stream) {
  int total = 0;
  int64_t bytes = 0;
  for (int j = 0; j < args.njobs; ++j) {
    args.job[j].block0 = total;
    total += args.job[j].nblocks;
    bytes += 2 * args.job[j].n;
  }
  const bool st = bytes >= kStreamBytes;
  if (args.in_f16 && st)
    hipLaunchKernelGGL((k_amax<true, true>), dim3(total), dim3(kAmaxThreads), 0, stream, args);
  else if (args.in_f16)
    hipLaunchKernelGGL((k_amax<false, true>), dim3(total), dim3(kAmaxThreads), 0, stream, args);
  else if (st)
    hipLaunchKernelGGL(k_amax<true>, dim3(total), dim3(kAmaxThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(k_amax<false>, dim3(total), dim3(kAmaxThreads), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !finalize) return e;
  hipLaunchKernelGGL(k_amax_finalize, dim3(args.njobs), dim3(kAmaxThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace fp8sg
