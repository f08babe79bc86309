// GradScaler step on the device [PT-CH20 §20.2.2: unscale the gradients, check
// them for inf/NaN, skip the optimizer step and shrink the scale when one is
// found; §20.5.33: the update() state machine; AMP-NOTES §4 steps 3-6].
//
// Unscale + check is one multi-tensor pass: the tensor list travels in the
// kernel arguments (up to kAmpTensorsPerLaunch tensors per launch, no device
// table to allocate or copy), every block owns 8192 consecutive elements of one
// tensor and finds its tensor by binary search over the per-tensor block
// offsets.  A tensor may start anywhere 2-byte aligned (views into a flat
// gradient bucket): the kernel walks the enclosing 16-byte-aligned span with
// 16-byte vectors and handles the partial first and last vectors element by
// element, never writing outside the tensor.  Each element is read and written once in place (2 + 2 bytes); the
// non-finite test runs on the stored fp16 result, (bits & 0x7FFF) >= 0x7C00,
// so it costs no extra traffic.  A wave that saw one sets the flag with a
// plain store of 1 (all writers store the same value).  The scale update is a
// single-lane kernel that keeps scale, tracker and flag on the device, so the
// step never synchronises the host.
#include "common.hpp"
#include "launch.hpp"

namespace fp8sg {

constexpr int kAmpThreads = 256;
constexpr int kAmpUnroll = 4;
constexpr int kAmpElemsPerBlock = kAmpThreads * 8 * kAmpUnroll;  // 8192
constexpr int kAmpTensorsPerLaunch = 64;

struct AmpTable {
  uint16_t* ptr[kAmpTensorsPerLaunch];    // 16-byte-aligned base at or below the tensor
  int64_t numel[kAmpTensorsPerLaunch];    // elements from ptr to the tensor's end
  int32_t head[kAmpTensorsPerLaunch];     // elements between ptr and the tensor's start (0..7)
  int32_t block0[kAmpTensorsPerLaunch + 1];  // prefix sum of blocks per tensor
  int32_t ntensors;
  const float* scale;
  int32_t* found_inf;
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// two fp16 in a dword -> unscaled two fp16, and whether either result is inf/NaN
__device__ __forceinline__ uint32_t unscale2(uint32_t w, float inv, bool& bad) {
  const h2 h = __builtin_bit_cast(h2, w);
  const float a = (float)h[0] * inv;
  const float b = (float)h[1] * inv;
  const h2 o = h2{(_Float16)a, (_Float16)b};
  const uint32_t r = __builtin_bit_cast(uint32_t, o);
  bad |= ((r & 0x7FFFu) >= 0x7C00u) | (((r >> 16) & 0x7FFFu) >= 0x7C00u);
  return r;
}

template <bool S>
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

  uint4 v[kAmpUnroll];
#pragma unroll
  for (int u = 0; u < kAmpUnroll; ++u) {
    const int64_t e = base + 8 * (int64_t)(u * kAmpThreads + tid);
    v[u] = (e >= first && e + 8 <= n) ? ld16<S>(g + e) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kAmpUnroll; ++u) {
    const int64_t e = base + 8 * (int64_t)(u * kAmpThreads + tid);
    if (e >= first && e + 8 <= n) {
      uint4 o;
      o.x = unscale2(v[u].x, inv, bad);
      o.y = unscale2(v[u].y, inv, bad);
      o.z = unscale2(v[u].z, inv, bad);
      o.w = unscale2(v[u].w, inv, bad);
      st16<S>(g + e, o);
    } else if (e < n && e + 8 > first) {
      // a partial vector at the tensor's start or end: only its own elements
      const int64_t i0 = e > first ? e : first, i1 = e + 8 < n ? e + 8 : n;
      for (int64_t i = i0; i < i1; ++i) {
        const float f = (float)__builtin_bit_cast(_Float16, g[i]) * inv;
        const uint16_t r = __builtin_bit_cast(uint16_t, (_Float16)f);
        bad |= (r & 0x7FFFu) >= 0x7C00u;
        g[i] = r;
      }
    }
  }
  if (__ballot(bad) != 0 && (tid & (kWave - 1)) == 0) *t.found_inf = 1;
}

hipError_t launch_unscale_check(uint16_t* const* grads, const int64_t* numel, int32_t ntensors,
                                const float* scale, int32_t* found_inf, hipStream_t stream) {
  for (int32_t t0 = 0; t0 < ntensors; t0 += kAmpTensorsPerLaunch) {
    AmpTable tab{};
    tab.scale = scale;
    tab.found_inf = found_inf;
    int32_t total = 0;
    const int32_t cnt = ntensors - t0 < kAmpTensorsPerLaunch ? ntensors - t0 : kAmpTensorsPerLaunch;
    for (int32_t i = 0; i < cnt; ++i) {
      const uintptr_t p = reinterpret_cast<uintptr_t>(grads[t0 + i]);
      const int32_t head = (int32_t)((p & 15u) >> 1);
      const int64_t n = numel[t0 + i] > 0 ? numel[t0 + i] + head : 0;  // span from the base
      tab.ptr[tab.ntensors] = reinterpret_cast<uint16_t*>(p & ~(uintptr_t)15);
      tab.numel[tab.ntensors] = n;
      tab.head[tab.ntensors] = head;
      tab.block0[tab.ntensors] = total;
      total += (int32_t)((n + kAmpElemsPerBlock - 1) / kAmpElemsPerBlock);
      ++tab.ntensors;
    }
    tab.block0[tab.ntensors] = total;
    if (total == 0) continue;
    if (4ll * kAmpElemsPerBlock * total >= kStreamBytes)  // 2 B read + 2 B written per element
      hipLaunchKernelGGL(k_unscale_check<true>, dim3(total), dim3(kAmpThreads), 0, stream, tab);
    else
      hipLaunchKernelGGL(k_unscale_check<false>, dim3(total), dim3(kAmpThreads), 0, stream, tab);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
