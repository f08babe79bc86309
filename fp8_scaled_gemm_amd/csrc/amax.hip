// amax = max_i |x_i| over bf16 tensors [FP8-TRAIN §2: x.float().abs().max()].
//
// One pass over HBM, 2 bytes per element.  |x| is compared as the unsigned
// integer bits & 0x7FFF: for non-negative IEEE values (inf and NaN included)
// integer order is numeric order, so the maximum is exact, order-free and
// NaN-propagating (every NaN pattern sits above +inf).  Two bf16 lanes per
// dword are reduced together with packed 16-bit max.  Stages: per-thread
// grid-stride loop over 16-byte loads -> wavefront shuffle -> LDS across the
// block's waves -> one atomic max per block into the record's accumulator; the
// last block to finish (atomic ticket) publishes rec->amax and re-zeroes the
// accumulator and ticket, so no separate clearing launch is needed.
//
// Several tensors can share one launch (the forward pass reduces x and W
// together): each job owns a contiguous range of blocks.
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxUnroll = 4;  // 16-byte loads in flight per thread per iteration

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pmax(uint32_t a, uint32_t b) {
  us2 r = __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b));
  return __builtin_bit_cast(uint32_t, r);
}

__global__ __launch_bounds__(kAmaxThreads) void k_amax(AmaxArgs args) {
  int j = 0;
#pragma unroll
  for (int t = 1; t < kMaxAmaxJobs; ++t)
    if (t < args.njobs && (int)blockIdx.x >= args.job[t].block0) j = t;
  const AmaxJob job = args.job[j];
  const int lb = (int)blockIdx.x - job.block0;
  const int tid = threadIdx.x;

  const uint4* xv = reinterpret_cast<const uint4*>(job.x);
  const int64_t nvec = job.n >> 3;
  const int64_t step = (int64_t)job.nblocks * kAmaxThreads * kAmaxUnroll;
  const uint32_t mask = 0x7FFF7FFFu;
  uint32_t m = 0;
  for (int64_t base = (int64_t)lb * kAmaxThreads * kAmaxUnroll + tid; base < nvec; base += step) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      int64_t k = base + (int64_t)u * kAmaxThreads;
      v[u] = k < nvec ? xv[k] : make_uint4(0, 0, 0, 0);
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

  uint32_t code = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
  uint32_t bits = code << 16;                  // the bf16 magnitude as fp32 bits
  if (bits > 0x7F800000u) bits = 0x7FC00000u;  // any NaN -> canonical NaN
  bits = wave_max_u32(bits);

  __shared__ uint32_t wmax[kAmaxThreads / kWave];
  __shared__ int last;
  if ((tid & (kWave - 1)) == 0) wmax[tid / kWave] = bits;
  __syncthreads();
  if (tid == 0) {
    uint32_t b = wmax[0];
#pragma unroll
    for (int w = 1; w < kAmaxThreads / kWave; ++w) b = wmax[w] > b ? wmax[w] : b;
    fp8sg_scale_rec* rec = job.rec;
    atomicMax(&rec->_acc, b);
    __threadfence();
    uint32_t ticket = atomicAdd(&rec->_ticket, 1u);
    last = (ticket == (uint32_t)job.nblocks - 1);
  }
  __syncthreads();
  if (last && tid == 0) {
    fp8sg_scale_rec* rec = job.rec;
    uint32_t fin = atomicMax(&rec->_acc, 0u);  // atomic read of the final maximum
    rec->amax = __uint_as_float(fin);
    rec->_acc = 0u;
    rec->_ticket = 0u;
  }
}

int amax_blocks_for(int64_t n) {
  int64_t nvec = n >> 3;
  int64_t per_block = (int64_t)kAmaxThreads * kAmaxUnroll;
  int64_t b = (nvec + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > kAmaxMaxBlocksPerJob) b = kAmaxMaxBlocksPerJob;
  return (int)b;
}

hipError_t launch_amax(AmaxArgs args, hipStream_t stream) {
  int total = 0;
  for (int j = 0; j < args.njobs; ++j) {
    args.job[j].block0 = total;
    total += args.job[j].nblocks;
  }
  hipLaunchKernelGGL(k_amax, dim3(total), dim3(kAmaxThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace fp8sg
