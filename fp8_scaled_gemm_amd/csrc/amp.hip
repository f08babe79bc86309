// GradScaler step on the device [PT-CH20 §20.2.2: unscale the gradients, check
// them for inf/NaN, skip the optimizer step and shrink the scale when one is
// found; §20.5.33: the update() state machine; AMP-NOTES §4 steps 3-6].
//
// Unscale + check is one multi-tensor pass: the tensor list travels in the
// kernel arguments (up to kAmpTensorsPerLaunch tensors and 2^23 blocks per
// launch, no device table to allocate or copy), every block owns 8192
// consecutive elements of one tensor and finds its tensor by binary search over
// the per-tensor block offsets.  A tensor may start anywhere 2-byte aligned
// (views into a flat gradient bucket): the kernel walks the enclosing
// 16-byte-aligned span with 16-byte vectors and handles the partial first and
// last vectors element by element, never writing outside the tensor.  Each
// element is read and written once in place (2 + 2 bytes); the non-finite test
// runs on the stored fp16 result, (bits & 0x7FFF) >= 0x7C00, so it costs no
// extra traffic.  A wave that saw one sets the flag with a
// plain store of 1 (all writers store the same value).  The scale update is a
// single-lane kernel that keeps scale, tracker and flag on the device, so the
// step never synchronises the host.
//
// With the gradient norm [AMP-NOTES §6 and MP-06 §四: gradient clipping runs
// on the unscaled gradients; its norm is the 2-norm of all elements together]
// the same pass also squares every stored unscaled value (exact in fp32 for
// fp16 inputs) and sums in fp32 in a fixed order: the 8 squares of each
// 16-byte load in turn, the thread's 4 load sums in turn, a fixed tree over
// the block; one slot per block of a caller workspace; two small kernels add
// the slots in fp64 in a fixed order.  The result is the same on every run.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kAmpThreads = 256;
constexpr int kAmpUnroll = 4;
constexpr int kAmpElemsPerBlock = kAmpThreads * 8 * kAmpUnroll;  // 8192
constexpr int kAmpTensorsPerLaunch = 64;
constexpr int kAmpWaves = kAmpThreads / kWave;

struct AmpTable {
  uint16_t* ptr[kAmpTensorsPerLaunch];    // 16-byte-aligned base at or below the tensor
  int64_t numel[kAmpTensorsPerLaunch];    // elements from ptr to the tensor's end
  int32_t head[kAmpTensorsPerLaunch];     // elements between ptr and the tensor's start (0..7)
  int32_t block0[kAmpTensorsPerLaunch + 1];  // prefix sum of blocks per tensor
  int32_t ntensors;
  const float* scale;
  int32_t* found_inf;
  float* parts;   // norm mode: one fp32 slot per block, from part0
  int64_t part0;
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// two fp16 in a dword -> unscaled two fp16, and whether either result is
// inf/NaN; with NORM the squares of the two stored results are added to ss
template <bool NORM>
__device__ __forceinline__ uint32_t unscale2(uint32_t w, float inv, bool& bad, float& ss) {
  const h2 h = __builtin_bit_cast(h2, w);
  const float a = fp32_value((float)h[0] * inv);
  const float b = fp32_value((float)h[1] * inv);
  const h2 o = h2{(_Float16)a, (_Float16)b};
  const uint32_t r = __builtin_bit_cast(uint32_t, o);
  bad |= ((r & 0x7FFFu) >= 0x7C00u) | (((r >> 16) & 0x7FFFu) >= 0x7C00u);
  if constexpr (NORM) {
    const float oa = (float)o[0], ob = (float)o[1];
    ss = ss + oa * oa;
    ss = ss + ob * ob;
  }
  return r;
}

template <bool S, bool NORM>
__global__ __launch_bounds__(kAmpThreads) void k_unscale_check(AmpTable t) {
  const int b = blockIdx.x;
  int lo = 0, hi = t.ntensors;  // block0[lo] <= b < block0[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (t.block0[mid] <= b) lo = mid; else hi = mid;
  }
  uint16_t* g = t.ptr[lo];
  const int64_t n = t.numel[lo];   // the tensor is [first, n) of g
  const int64_t first = t.head[lo];
  const int64_t base = (int64_t)(b - t.block0[lo]) * kAmpElemsPerBlock;
  const float inv = 1.0f / *t.scale;
  const int tid = threadIdx.x;
  bool bad = false;
  float ssu[kAmpUnroll] = {};  // norm: one running sum per load of the thread

  // All loads issued with no branch between them (a branch or a select here
  // makes the compiler wait for the first loads before issuing the rest): a
  // lane without a whole vector of the tensor loads the 16-byte chunk at g,
  // which holds the tensor's first element (every block's tensor is
  // non-empty), and never uses it.
  uint4 v[kAmpUnroll];
#pragma unroll
  for (int u = 0; u < kAmpUnroll; ++u) {
    const int64_t e = base + 8 * (int64_t)(u * kAmpThreads + tid);
    v[u] = ld16<S>(g + ((e >= first && e + 8 <= n) ? e : 0));
  }
#pragma unroll
  for (int u = 0; u < kAmpUnroll; ++u) keep_loaded(v[u]);
#pragma unroll
  for (int u = 0; u < kAmpUnroll; ++u) {
    const int64_t e = base + 8 * (int64_t)(u * kAmpThreads + tid);
    if (e >= first && e + 8 <= n) {
      uint4 o;
      o.x = unscale2<NORM>(v[u].x, inv, bad, ssu[u]);
      o.y = unscale2<NORM>(v[u].y, inv, bad, ssu[u]);
      o.z = unscale2<NORM>(v[u].z, inv, bad, ssu[u]);
      o.w = unscale2<NORM>(v[u].w, inv, bad, ssu[u]);
      st16<S>(g + e, o);
    } else if (e < n && e + 8 > first) {
      // a partial vector at the tensor's start or end: only its own elements
      const int64_t i0 = e > first ? e : first, i1 = e + 8 < n ? e + 8 : n;
      for (int64_t i = i0; i < i1; ++i) {
        const float f = fp32_value((float)__builtin_bit_cast(_Float16, g[i]) * inv);
        const _Float16 o = (_Float16)f;
        const uint16_t r = __builtin_bit_cast(uint16_t, o);
        bad |= (r & 0x7FFFu) >= 0x7C00u;
        if constexpr (NORM) ssu[u] = ssu[u] + (float)o * (float)o;
        g[i] = r;
      }
    }
  }
  if (__ballot(bad) != 0 && (tid & (kWave - 1)) == 0) *t.found_inf = 1;
  if constexpr (NORM) {
    // the thread's sums in order, xor-shuffles inside each wave, then the four
    // wave sums in order
    float ss = ssu[0];
#pragma unroll
    for (int u = 1; u < kAmpUnroll; ++u) ss = ss + ssu[u];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) ss = ss + __shfl_xor(ss, off, kWave);
    __shared__ float wsum[kAmpWaves];
    if ((tid & (kWave - 1)) == 0) wsum[tid / kWave] = ss;
    __syncthreads();
    if (tid == 0) {
      float tot = wsum[0];
#pragma unroll
      for (int w = 1; w < kAmpWaves; ++w) tot = tot + wsum[w];
      t.parts[t.part0 + b] = tot;
    }
  }
}

// Sum of the per-block slots in fp64, in a fixed order, in two stages.
// Stage 1: block g of kNormGroups adds slots [g c, g c + c), c = ceil(n / G):
// thread i adds slots g c + i, + 256, ... in turn (8 loads in flight), then a
// fixed tree over the block, into fp64 partial g.  Stage 2: one block adds the
// G partials the same way and writes out[0] = the sum rounded to fp32,
// out[1] = its square root (fp64, rounded to fp32).
constexpr int kNormGroups = 256;

__device__ __forceinline__ double block_sum_f64(double s) {
  __shared__ double red[kAmpThreads];
  const int tid = threadIdx.x;
  red[tid] = s;
  __syncthreads();
#pragma unroll
  for (int h = kAmpThreads / 2; h > 0; h >>= 1) {
    if (tid < h) red[tid] = red[tid] + red[tid + h];
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(kAmpThreads) void k_norm_partial(const float* parts, int64_t n,
                                                               double* part64) {
  const int64_t c = (n + kNormGroups - 1) / kNormGroups;
  const int64_t lo = (int64_t)blockIdx.x * c, hi = lo + c < n ? lo + c : n;
  double s = 0.0;
  constexpr int kIn = 8;
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)kIn * kAmpThreads) {
    float v[kIn];
#pragma unroll
    for (int q = 0; q < kIn; ++q) {
      const int64_t k = i + (int64_t)q * kAmpThreads;
      v[q] = k < hi ? parts[k] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kIn; ++q) s = s + (double)v[q];
  }
  s = block_sum_f64(s);
  if (threadIdx.x == 0) part64[blockIdx.x] = s;
}

__global__ __launch_bounds__(kAmpThreads) void k_norm_finalize(const double* part64, float* out) {
  double s = threadIdx.x < kNormGroups ? part64[threadIdx.x] : 0.0;
  s = block_sum_f64(s);
  if (threadIdx.x == 0) {
    out[0] = (float)s;
    out[1] = (float)__builtin_sqrt(s);
  }
}

static int64_t unscale_blocks(uint16_t* const* grads, const int64_t* numel, int32_t ntensors) {
  int64_t total = 0;
  for (int32_t i = 0; i < ntensors; ++i) {
    const int64_t head = (int64_t)((reinterpret_cast<uintptr_t>(grads[i]) & 15u) >> 1);
    const int64_t n = numel[i] > 0 ? numel[i] + head : 0;
    total += (n + kAmpElemsPerBlock - 1) / kAmpElemsPerBlock;
  }
  return total;
}

// Workspace (in floats): one slot per block, then kNormGroups fp64 partials
// at the next 8-byte boundary.
static int64_t norm_ws_len(int64_t blocks) { return ((blocks + 1) & ~int64_t(1)) + 2 * kNormGroups; }

int64_t norm_slots(uint16_t* const* grads, const int64_t* numel, int32_t ntensors) {
  return norm_ws_len(unscale_blocks(grads, numel, ntensors));
}

int64_t unscale_blocks_bound(const int64_t* numel, int32_t ntensors) {
  int64_t total = 0;
  for (int32_t i = 0; i < ntensors; ++i)
    if (numel[i] > 0) total += (numel[i] + 7 + kAmpElemsPerBlock - 1) / kAmpElemsPerBlock;
  return norm_ws_len(total);
}

hipError_t launch_unscale_check(uint16_t* const* grads, const int64_t* numel, int32_t ntensors,
                                const float* scale, int32_t* found_inf, float* parts,
                                float* sumsq_norm, hipStream_t stream) {
  // A launch takes up to kAmpTensorsPerLaunch tensors and kAmpMaxBlocks
  // blocks; a tensor of at most FP8SG_MAX_ELEMS elements always fits alone.
  constexpr int32_t kAmpMaxBlocks = 1 << 23;
  static_assert(FP8SG_MAX_ELEMS / kAmpElemsPerBlock + 1 <= kAmpMaxBlocks, "one tensor per launch");
  int64_t part0 = 0;
  AmpTable tab{};
  int32_t total = 0;
  auto flush = [&]() -> hipError_t {
    tab.block0[tab.ntensors] = total;
    if (total > 0) {
      tab.scale = scale;
      tab.found_inf = found_inf;
      tab.parts = parts;
      tab.part0 = part0;
      const bool stream_pass = 4ll * kAmpElemsPerBlock * total >= kStreamBytes;  // 2 B in + 2 B out
      if (parts && stream_pass)
        hipLaunchKernelGGL((k_unscale_check<true, true>), dim3(total), dim3(kAmpThreads), 0, stream, tab);
      else if (parts)
        hipLaunchKernelGGL((k_unscale_check<false, true>), dim3(total), dim3(kAmpThreads), 0, stream, tab);
      else if (stream_pass)
        hipLaunchKernelGGL((k_unscale_check<true, false>), dim3(total), dim3(kAmpThreads), 0, stream, tab);
      else
        hipLaunchKernelGGL((k_unscale_check<false, false>), dim3(total), dim3(kAmpThreads), 0, stream, tab);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      part0 += total;
    }
    tab = AmpTable{};
    total = 0;
    return hipSuccess;
  };
  for (int32_t i = 0; i < ntensors; ++i) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(grads[i]);
    const int32_t head = (int32_t)((p & 15u) >> 1);
    const int64_t n = numel[i] > 0 ? numel[i] + head : 0;  // span from the base
    const int32_t nb = (int32_t)((n + kAmpElemsPerBlock - 1) / kAmpElemsPerBlock);
    if (tab.ntensors == kAmpTensorsPerLaunch || total + (int64_t)nb > kAmpMaxBlocks) {
      const hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
    tab.ptr[tab.ntensors] = reinterpret_cast<uint16_t*>(p & ~(uintptr_t)15);
    tab.numel[tab.ntensors] = n;
    tab.head[tab.ntensors] = head;
    tab.block0[tab.ntensors] = total;
    total += nb;
    ++tab.ntensors;
  }
  const hipError_t ef = flush();
  if (ef != hipSuccess) return ef;
  if (parts) {
    double* part64 = reinterpret_cast<double*>(parts + ((part0 + 1) & ~int64_t(1)));
    hipLaunchKernelGGL(k_norm_partial, dim3(kNormGroups), dim3(kAmpThreads), 0, stream, parts,
                       part0, part64);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_norm_finalize, dim3(1), dim3(kAmpThreads), 0, stream, part64, sumsq_norm);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Scratch of the norm pass for callers that cannot allocate: a fixed device
// array in place of the caller's workspace, one copy per GPU, held until the
// process ends.  Its address on a device comes from hipGetSymbolAddress, taken
// once per device with that device current; host code uses only that address
// (the array's name in host code is not a device address).  Every slot the
// pass reads was written earlier in the same call (the per-block slots by the
// unscale kernel, the fp64 partials by the first sum kernel), so nothing needs
// clearing between calls; calls that overlap in time on one GPU share it and
// race.
static __device__ __align__(256) float scratch[kNoAllocNormSlots];

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static float* g_scratch[kMaxScratchDevices] = {};

hipError_t norm_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// GradScaler.update() [PT-CH20 §20.5.33], then the flag is cleared for the next step.
__global__ void k_update_scale(float* scale, int32_t* tracker, int32_t* found_inf, float growth,
                               float backoff, int32_t interval) {
  if (threadIdx.x != 0) return;
  float s = *scale;
  int32_t t = *tracker;
  if (*found_inf) {
    s = s * backoff;
    t = 0;
  } else {
    t = t + 1;
    if (t >= interval) {
      s = s * growth;
      t = 0;
    }
  }
  *scale = s;
  *tracker = t;
  *found_inf = 0;
}

hipError_t launch_update_scale(float* scale, int32_t* tracker, int32_t* found_inf, float growth,
                               float backoff, int32_t interval, hipStream_t stream) {
  hipLaunchKernelGGL(k_update_scale, dim3(1), dim3(kWave), 0, stream, scale, tracker, found_inf,
                     growth, backoff, interval);
  return hipGetLastError();
}

}  // namespace fp8sg
