// Host-side launch interface between the C-ABI layer (api.hip) and the kernel
// translation units.  Kernel arguments travel by value (no device tables), so a
// launch needs no allocation and no host-to-device copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8sg.h"

namespace fp8sg {

// ---- amax (amax.hip)
constexpr int kMaxAmaxJobs = 4;

struct AmaxJob {
  const uint16_t* x;
  int64_t n;
  fp8sg_scale_rec* rec;
  int32_t block0;   // first block of this job (filled by launch_amax)
  int32_t nblocks;  // blocks given to this job (amax_blocks_for, <= FP8SG_AMAX_PARTS)
};
struct AmaxArgs {
  AmaxJob job[kMaxAmaxJobs];
  int32_t njobs;
  int32_t in_f16;  // inputs are fp16 (default: bf16)
};
int amax_blocks_for(int64_t n);
// Per-block partial maxima into each job's record; with finalize, also rec->amax.
hipError_t launch_amax(AmaxArgs args, bool finalize, hipStream_t stream);

// ---- quantize (quantize.hip)
constexpr int kMaxQuantJobs = 4;

struct QuantJob {
  const uint16_t* x;
  int64_t rows, cols;
  fp8sg_scale_rec* rec;
  uint8_t* q;
  uint8_t* qT;      // may be null
  int32_t block0;   // filled by the launcher
  int32_t nblocks;
  int32_t tiles_c;  // tiled path: tiles along cols
  float* hist;      // delayed scaling: amax history (most recent first), or null
  int32_t hist_len;
  const float* amax_in;  // the caller's amax (device fp32), or null; never with hist
};
struct QuantArgs {
  QuantJob job[kMaxQuantJobs];
  int32_t njobs;
  int32_t in_f16;  // inputs are fp16 (default: bf16); dynamic scaling only
};
// All jobs of one launch share the format.  Chooses the tiled kernel (rows and
// cols multiples of 16 with a transposed copy), the flat kernel (no transposed
// copy) or the per-element kernel (a transposed copy of an odd shape).
hipError_t launch_quantize(QuantArgs args, int fmt, hipStream_t stream);
// Small tensors: one block per job reduces its own amax and casts it, so the
// amax launch is not needed (tiled path, dynamic scaling, at most
// kSelfCastMaxElems elements per job).  Records, codes and transposed codes
// as launch_amax + launch_quantize write them.
constexpr int64_t kSelfCastMaxElems = 65536;
bool self_cast_fits(const QuantArgs& a);
hipError_t launch_quantize_self(QuantArgs args, int fmt, hipStream_t stream);

// ---- GEMM (gemm.hip)
struct GemmProblem {
  const uint8_t* A;
  const uint8_t* B;
  void* C;
  const double* inv_a;
  const double* inv_b;
  int64_t M, N, K;
  const float* amp_scale;  // kOutF16Unscale only: the GradScaler's loss scale
  int32_t* found_inf;      // kOutF16Unscale only: set to 1 on a non-finite output
};
// Internal output mode next to fp8sg_out: fp16 output h = fp16(acc * alpha),
// then unscaled in the epilogue as the GradScaler does it, g = fp16(fl32(h) *
// fl32(1 / *amp_scale)), with found_inf set when a stored g is inf or NaN.
constexpr int kOutF16Unscale = 3;
hipError_t launch_gemm(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream);
// Contraction-major operands (gemm_km*.hip): ta / tb mean A is stored as
// A^T [K, M] / B as B^T [K, N], row-major; out may be kOutF16Unscale.  The
// pair is a linear layer's backward without transposed copies: dgrad
// (gy codes, W codes as B^T) and wgrad (gy codes as A^T, x codes as B^T),
// e5m2 x e4m3.
hipError_t launch_gemm_km(const GemmProblem& p, int fa, int fb, int out, bool ta, bool tb,
                          hipStream_t stream);
hipError_t launch_gemm_km_pair(const GemmProblem& dgrad, const GemmProblem& wgrad, int out,
                               hipStream_t stream);
// Which transposed copies make the backward of an M x N x K linear layer
// fastest on the current device (fp8_linear_copies).
void linear_copies(int64_t M, int64_t N, int64_t K, bool& x_t, bool& w_t, bool& gy_t);

// Small layers in one launch per pass (small_layer.hip), for layers whose x,
// W and gy each hold at most kSelfCastMaxElems elements and that keep no
// transposed copies.  Forward: p is the forward GEMM (A = x_q, B = w_q, C = y;
// its inverse pointers are not read), x and w the bf16 inputs.  Backward: dg
// and wg are the dgrad and wgrad problems on contraction-major codes (their
// inv_b point to the saved records' inverses), gy the bf16 gradient
// [rows, cols].
struct SmallFwdArgs {
  const uint16_t* x;
  const uint16_t* w;
  GemmProblem p;
  fp8sg_scale_rec* x_sc;
  fp8sg_scale_rec* w_sc;
  uint8_t* x_q;
  uint8_t* w_q;
};
struct SmallBwdArgs {
  const uint16_t* gy;
  int64_t rows, cols;
  GemmProblem dg, wg;
  fp8sg_scale_rec* gy_sc;
  uint8_t* gy_q;
};
bool small_layer_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_small_fwd(const SmallFwdArgs& a, int out, hipStream_t stream);
hipError_t launch_small_bwd(const SmallBwdArgs& a, int out, hipStream_t stream);
// Row-wise scaling (gemm_rowwise.hip): inv_a points to M doubles, inv_b to N;
// element (m, n) is scaled by fl32(inv_a[m] * inv_b[n]).
hipError_t launch_gemm_rowwise(const GemmProblem& p, int fa, int fb, int out, hipStream_t stream);
// The kOutF16Unscale epilogue (gemm_unscale.hip); p.amp_scale and p.found_inf set.
hipError_t launch_gemm_unscale(const GemmProblem& p, int fa, int fb, hipStream_t stream);
// The backward pair (dgrad, wgrad): one launch of the 128 x 128 kernel when
// both are small, otherwise one launch each.
hipError_t launch_gemm_pair(const GemmProblem& p0, const GemmProblem& p1, int fa, int fb, int out,
                           hipStream_t stream);
// The backward pair with the fused unscale; rowwise selects the row-wise
// epilogue factors (GemmProblem's inverse pointers are then vectors).
hipError_t launch_gemm_unscale_pair(const GemmProblem& p0, const GemmProblem& p1, bool rowwise,
                                    hipStream_t stream);
hipError_t launch_gemm_rowwise_pair(const GemmProblem& p0, const GemmProblem& p1, int out,
                                    hipStream_t stream);

// ---- row-wise quantize (rowwise.hip)
struct RowwiseArgs {
  const uint16_t* x;
  int64_t rows, cols;  // multiples of 16
  float* row_amax;     // [rows]
  double* row_inv;     // [rows]
  uint8_t* q;          // [rows, cols], codes with the row scales
  float* col_amax;     // [cols] (with qT)
  double* col_inv;     // [cols] (with qT)
  uint8_t* qT;         // [cols, rows], codes with the column scales; may be null
  int32_t tiles_c;     // filled by the launcher
};
// Three launches: per-tile partial maxima (stored in q's memory), their
// reduction into the amax / inverse-scale vectors, the cast.
hipError_t launch_rowwise(const RowwiseArgs& a, int fmt, hipStream_t stream);
// Two casts in the same three launches (x and W of a layer); falls back to
// one cast after the other when either is empty or only one has a qT.
hipError_t launch_rowwise2(const RowwiseArgs& a0, const RowwiseArgs& a1, int fmt,
                           hipStream_t stream);

// ---- GradScaler (amp.hip)
// Norm workspace slots of the unscale pass for these tensors (exact; needs the
// pointers' alignment) and an upper bound that needs only the sizes.
int64_t norm_slots(uint16_t* const* grads, const int64_t* numel, int32_t ntensors);
int64_t unscale_blocks_bound(const int64_t* numel, int32_t ntensors);
// parts == nullptr: unscale + check only; otherwise also one sum-of-squares
// slot per block in parts and the finalized (sum, norm) in sumsq_norm.
hipError_t launch_unscale_check(uint16_t* const* grads, const int64_t* numel, int32_t ntensors,
                                const float* scale, int32_t* found_inf, float* parts,
                                float* sumsq_norm, hipStream_t stream);
// The norm pass's scratch for amp_unscale_check_norm_noalloc: a static device
// array of kNoAllocNormSlots floats (4 MiB) per GPU; *out is its address on the
// current device (looked up once per device).
constexpr int64_t kNoAllocNormSlots = FP8SG_NOALLOC_NORM_SLOTS;
hipError_t norm_scratch(float** out);
hipError_t launch_update_scale(float* scale, int32_t* tracker, int32_t* found_inf, float growth,
                               float backoff, int32_t interval, hipStream_t stream);

}  // namespace fp8sg
