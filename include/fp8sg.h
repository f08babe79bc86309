/*
 * fp8sg -- FP8 per-tensor dynamically scaled linear layer and GradScaler step
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operations follow these web pages (cited by title and section):
 *   [FP8-TRAIN]  "FP8训练：量化、自动微分、Torchao" (lzwjava.github.io)
 *   [PT-CH20]    "第20章 量化与混合精度训练" (yangyitao.com, PyTorch book ch. 20)
 *   [AMP-MP]     "从 AMP 到 Mixed Precision" (111qqz.com)
 *   [AMP-NOTES]  "AMP：Automatic Mixed Precision 技术笔记" (luna-shi.github.io)
 *
 * Conventions shared by every entry point:
 *  - All tensor and state pointers are DEVICE pointers into memory the caller
 *    owns; the library allocates no device memory on any of these calls.
 *    Host pointers appear only where a parameter says "host".
 *  - Element types are passed as their bit patterns: bf16 and fp16 as
 *    uint16_t, FP8 codes as uint8_t.  Matrices are row-major and contiguous.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    validates its arguments and enqueues kernels on `stream`; it never
 *    synchronises the host.  Results are ready when the stream's work is.
 *  - Errors: argument errors are reported before anything is enqueued
 *    (FP8SG_ERR_NULL, _SHAPE, _ALIGN, _FORMAT).  FP8SG_ERR_HIP means a launch
 *    failed; kernels already enqueued by the call may have run.  No exception
 *    crosses the ABI, and there is no global error state besides the return.
 *  - Device pointers to tensors must be 16-byte aligned (FP8SG_ERR_ALIGN),
 *    except the fp16 gradients of amp_unscale_check (2-byte aligned); scale
 *    records 8-byte aligned; fp32 and int32 scalars 4-byte aligned.
 *  - Sizes are bounded by FP8SG_MAX_DIM and FP8SG_MAX_ELEMS (below).
 *  - Calls that share an output or state buffer must not overlap in time.
 */
#ifndef FP8SG_H
#define FP8SG_H

#include <stdint.h>

#if defined(__GNUC__)
#define FP8SG_API __attribute__((visibility("default")))
#else
#define FP8SG_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8SG_E4M3FN = 0, /* 1|4|3, bias 7, no inf, largest 448 [FP8-TRAIN §2, §3]  */
  FP8SG_E5M2 = 1    /* 1|5|2, bias 15, IEEE-style inf/NaN, largest 57344 [§3] */
} fp8sg_format;

typedef enum {
  FP8SG_OUT_BF16 = 0, /* bf16, round-to-nearest-even (the layer's dtype)  */
  FP8SG_OUT_F16 = 1,  /* fp16, round-to-nearest-even (fp16 AMP gradients) */
  FP8SG_OUT_F32 = 2   /* fp32, unrounded epilogue value                   */
} fp8sg_out;

typedef enum {
  FP8SG_OK = 0,
  FP8SG_ERR_NULL = 1,   /* a required pointer is NULL                      */
  FP8SG_ERR_SHAPE = 2,  /* a size is negative, above the size limits below
                           or breaks a multiple-of rule                     */
  FP8SG_ERR_ALIGN = 3,  /* a pointer lacks the alignment its call needs:
                           16 bytes for tensors, 8 for scale records and
                           fp64 vectors, 4 for fp32/int32 scalars           */
  FP8SG_ERR_FORMAT = 4, /* unknown fp8sg_format / fp8sg_out value          */
  FP8SG_ERR_HIP = 5     /* a HIP launch or runtime call failed             */
} fp8sg_status;

typedef void* fp8sg_stream; /* hipStream_t */

/* Number of per-block partial maxima an amax reduction leaves in a record. */
#define FP8SG_AMAX_PARTS 1024
/* Longest amax history the delayed-scaling entry points take. */
#define FP8SG_MAX_HISTORY 1024

/*
 * Size limits, checked by every entry point (FP8SG_ERR_SHAPE beyond them).
 * A matrix dimension (rows and cols of a row-wise cast, M, N, Kc of a GEMM or
 * linear layer) is at most FP8SG_MAX_DIM; every tensor an entry point reads
 * or writes holds at most FP8SG_MAX_ELEMS elements (64 GiB of bf16).  The
 * launch grids and 32-bit per-launch block counts are sized for these.
 * fp8_amax, fp8_quantize, fp8_quantize_delayed and the amp_* calls bound only
 * the element count.
 */
#define FP8SG_MAX_DIM (1LL << 29)
#define FP8SG_MAX_ELEMS (1LL << 35)

/*
 * Per-tensor scale record, 4128 bytes of device memory owned by the caller
 * [FP8-TRAIN §2]: the tensor's absolute maximum, the fp64 scale
 * fp8_max / max(amax, EPS) with EPS = 1e-12, its fp64 reciprocal (the inverse
 * the GEMM dequantises with) and both rounded to fp32 (the quantizer
 * multiplies by scale32).  The underscore fields hold the amax reduction's
 * per-block partial maxima, written by fp8_amax and read by fp8_quantize; no
 * initialisation is needed.
 */
typedef struct fp8sg_scale_rec {
  float amax;        /* max_i |x_i| as fp32; canonical NaN 0x7FC00000 if any NaN */
  float scale32;     /* (float)scale                                             */
  float inv32;       /* (float)inv                                               */
  uint32_t _nparts;  /* library-internal: partial maxima in _part                */
  double scale;      /* fp8_max / max(amax, EPS), IEEE fp64 division             */
  double inv;        /* 1.0 / scale, IEEE fp64 division                          */
  uint32_t _part[FP8SG_AMAX_PARTS]; /* library-internal: per-block maxima (fp32 bits) */
} fp8sg_scale_rec;

/* Human-readable name of a status code (static storage). */
FP8SG_API const char* fp8sg_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
FP8SG_API int fp8sg_version(void);

/*
 * amax of a bf16 tensor [FP8-TRAIN §2: x.float().abs().max()].
 *   x:   n bf16 values (device, 16-byte aligned; may be NULL when n == 0);
 *        n >= 0, any n.
 *   rec: scale record (device); writes rec->amax and the partial maxima.
 *        n == 0 gives +0.
 * A NaN anywhere gives the canonical NaN; +-inf gives +inf.
 */
FP8SG_API fp8sg_status fp8_amax(const uint16_t* x, int64_t n, fp8sg_scale_rec* rec, fp8sg_stream stream);

/*
 * Scale and quantize-cast of a bf16 matrix [FP8-TRAIN §2 (scale in fp64,
 * x*scale, clamp to +-fp8_max, cast), §3 (e4m3 for activations and weights,
 * e5m2 for gradients), §4 (the transposed copy the backward GEMMs need)].
 *   x:    rows x cols bf16, row-major (device, 16-byte aligned).
 *   fmt:  FP8SG_E4M3FN or FP8SG_E5M2.
 *   rec:  scale record filled by fp8_amax on this same tensor x, with no other
 *         call on rec in between; this call reduces the partial maxima fp8_amax
 *         left there and writes amax, scale, inv, scale32 and inv32.  The
 *         partials are the only input the scale is taken from: a record
 *         reduced over another tensor gives that tensor's scale, without an
 *         error.  A caller holding the amax itself uses fp8_quantize_from_amax.
 *   q:    rows x cols codes, row-major (device, 16-byte aligned).
 *   qT:   cols x rows codes = transpose of q (device, 16-byte aligned), or
 *         NULL to skip the transposed copy.
 * Each code is enc(clamp(fl32(x * scale32), -max, max)) rounded to nearest
 * even; NaN inputs give a NaN code.  rows, cols >= 0 (x, q, qT may be NULL
 * when rows * cols == 0; the record's scale fields are still written).  With
 * qT, rows and cols that are multiples of 16 take the tiled fast path; other
 * shapes are handled by a plain per-element kernel.
 */
FP8SG_API fp8sg_status fp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, fp8sg_format fmt,
                          fp8sg_scale_rec* rec, uint8_t* q, uint8_t* qT, fp8sg_stream stream);

/*
 * fp8_amax and fp8_quantize for fp16 tensors: the same definitions [FP8-TRAIN
 * §2] with an fp16 input (x as fp16 bit patterns, decoded exactly to fp32), for
 * a model kept in fp16 under loss scaling [PT-CH20 §20.2.2].  The record,
 * codes, transposed codes, limits and errors are as for the bf16 calls; a NaN
 * anywhere gives the canonical NaN amax, +-inf gives +inf.  The record pairs
 * the two calls as it pairs fp8_amax and fp8_quantize.
 */
FP8SG_API fp8sg_status fp8_amax_f16(const uint16_t* x, int64_t n, fp8sg_scale_rec* rec,
                                    fp8sg_stream stream);
FP8SG_API fp8sg_status fp8_quantize_f16(const uint16_t* x, int64_t rows, int64_t cols,
                                        fp8sg_format fmt, fp8sg_scale_rec* rec, uint8_t* q,
                                        uint8_t* qT, fp8sg_stream stream);

/*
 * fp8_quantize with the amax supplied by the caller [FP8-TRAIN §2: the scale
 * is fp8_max / amax in fp64, then x * scale, clamp, cast].  The scale, inverse
 * and codes are those fp8_quantize computes from a record whose amax is *amax;
 * nothing is read from rec before it is written, so rec needs no fp8_amax.
 * This is the call for an amax that was combined outside this tensor: the
 * maximum over the shards of a tensor split across devices (a MAX all-reduce of
 * the shards' fp8_amax results) or an amax the caller tracks itself.
 *   amax: device float (4-byte aligned), read on `stream`.  NaN gives the NaN
 *         scale; a negative value counts as 0.  rec->amax receives the value
 *         used (canonical NaN, or +0 for a negative input).
 *   rec:  scale record (device): amax, scale, inv, scale32 and inv32 written.
 * The other arguments, layouts and the transposed copy as fp8_quantize.
 */
FP8SG_API fp8sg_status fp8_quantize_from_amax(const uint16_t* x, int64_t rows, int64_t cols,
                                    fp8sg_format fmt, const float* amax, fp8sg_scale_rec* rec,
                                    uint8_t* q, uint8_t* qT, fp8sg_stream stream);

/*
 * Scaled FP8 GEMM [FP8-TRAIN §2, §4; AMP-MP "不要忘记 Accumulator Precision"]:
 *   C[M,N] = out( (sum_k dec(A[m,k]) * dec(B[n,k])) * fl32(inv_a * inv_b) )
 * with the sum accumulated in fp32 (any order) and the product of the two
 * fp64 inverse scales rounded once to fp32.
 *   A:  M x Kc codes of format fa, row-major (contiguous along Kc).
 *   B:  N x Kc codes of format fb, row-major (contiguous along Kc).
 *   inv_a, inv_b: device doubles, 8-byte aligned (e.g. &rec->inv).
 *   C:  M x N of type `out`, row-major.
 *   M, N, Kc >= 0 and multiples of 16 (FP8SG_ERR_SHAPE otherwise).  Kc == 0
 *   gives C = 0 * alpha.  A pointer to a zero-sized operand may be NULL.
 */
FP8SG_API fp8sg_status fp8_gemm(const uint8_t* A, fp8sg_format fa, const uint8_t* B, fp8sg_format fb,
                      const double* inv_a, const double* inv_b, void* C, fp8sg_out out,
                      int64_t M, int64_t N, int64_t Kc, fp8sg_stream stream);

/*
 * fp8_gemm into fp16 with the GradScaler's unscale and non-finite check
 * fused into the epilogue [PT-CH20 §20.2.2; FP8-TRAIN §4]: each element is
 *   h = fp16(acc * fl32(inv_a * inv_b)),  C = fp16(fl32(h) * fl32(1.0f / *scale))
 * (both fp16 roundings to nearest even, as fp8_gemm with FP8SG_OUT_F16 followed
 * by amp_unscale_check on C), and *found_inf is set to 1 (never cleared) if a
 * stored C element is inf or NaN.
 *   scale: device float (4-byte aligned); found_inf: device int32.
 *   C: M x N fp16 bit patterns.  The other arguments as fp8_gemm.
 */
FP8SG_API fp8sg_status fp8_gemm_unscale(const uint8_t* A, fp8sg_format fa, const uint8_t* B,
                              fp8sg_format fb, const double* inv_a, const double* inv_b,
                              const float* scale, int32_t* found_inf, uint16_t* C, int64_t M,
                              int64_t N, int64_t Kc, fp8sg_stream stream);

/*
 * Scaled FP8 GEMM with contraction-major operands [FP8-TRAIN §4 backward: the
 * dgrad and wgrad products contract x, W and gy over their other dimension].
 * As fp8_gemm, except that with a_kmajor != 0 A is stored as A^T: Kc x M
 * codes, row-major (contiguous along M); with b_kmajor != 0 B is stored as
 * B^T: Kc x N, row-major.  The kernels read such an operand in its own layout
 * (LDS transpose reads), so the backward GEMMs of a linear layer can use the
 * row-major codes of x, W and gy instead of transposed copies:
 *   dgrad gx = gy W:   fp8_gemm_kmajor(gy_q, e5m2, 0, w_q, e4m3, 1, ..., M, K, N)
 *   wgrad gW = gy^T x: fp8_gemm_kmajor(gy_q, e5m2, 1, x_q, e4m3, 1, ..., N, K, M)
 * The products and their summation order are those of fp8_gemm on the
 * transposed copies, so the results are the same bits.  Shapes, alignment,
 * errors and the unscale variant's extra arguments as fp8_gemm and
 * fp8_gemm_unscale.
 */
FP8SG_API fp8sg_status fp8_gemm_kmajor(const uint8_t* A, fp8sg_format fa, int32_t a_kmajor,
                                       const uint8_t* B, fp8sg_format fb, int32_t b_kmajor,
                                       const double* inv_a, const double* inv_b, void* C,
                                       fp8sg_out out, int64_t M, int64_t N, int64_t Kc,
                                       fp8sg_stream stream);
FP8SG_API fp8sg_status fp8_gemm_kmajor_unscale(const uint8_t* A, fp8sg_format fa, int32_t a_kmajor,
                                               const uint8_t* B, fp8sg_format fb, int32_t b_kmajor,
                                               const double* inv_a, const double* inv_b,
                                               const float* scale, int32_t* found_inf, uint16_t* C,
                                               int64_t M, int64_t N, int64_t Kc,
                                               fp8sg_stream stream);

/*
 * What the forward pass saves for the backward pass [FP8-TRAIN §6: the
 * quantized FP8 tensors and their inverse scales, not the bf16 inputs].
 * All pointers are caller-owned device buffers.  Each transposed copy (x_qT,
 * w_qT here, gy_qT in the workspace) may be NULL on its own: that copy is not
 * made, and the backward GEMM that would read it reads the row-major codes
 * contraction-major instead (fp8_gemm_kmajor).  Every combination gives the
 * same results bit for bit; a cast without its copy writes 1 B per element
 * instead of 2.  Speed: a contraction-major operand costs nothing in the
 * GEMM's second (B) slot and about 8% in the first (A) slot, which takes
 * twice the fragment reads.  dgrad reads W in the B slot; wgrad gW = gy^T x
 * puts gy in the A slot, except where the launcher swaps the roles to fit
 * 224-row tiles along K (then x takes the A slot: the MLP block's
 * down-projection, N = 4096, K = 14336).  Keeping the copy of the A-slot
 * operand only is the fastest form where the layer is large.
 */
/*
 * Which transposed copies make the backward GEMMs of a linear layer with
 * these sizes fastest on the current device [FP8-TRAIN §4: dgrad and wgrad
 * contract x, W and gy over their other dimension]; the results are the same
 * bits with any choice (see fp8_linear_saved below).  A copy costs its cast
 * one more byte written per element, which this choice does not weigh.
 *   M tokens, N outputs, K inputs: > 0, multiples of 16 (FP8SG_ERR_SHAPE).
 *   *x_T, *w_T, *gy_T: 1 = make that copy, 0 = read the row-major codes
 *   contraction-major.  W never needs one (dgrad reads it in the GEMM's
 *   second slot); of x and gy, the weight gradient's first-slot operand keeps
 *   its copy when that GEMM takes the 256 x 256 (or 224-row) kernel; small
 *   layers keep none.  Host-only: queries the device's CU count, launches
 *   nothing.
 */
FP8SG_API fp8sg_status fp8_linear_copies(int64_t M, int64_t N, int64_t K, int32_t* x_T,
                                         int32_t* w_T, int32_t* gy_T);

typedef struct fp8_linear_saved {
  uint8_t* x_q;         /* [M,K] e4m3 codes of x                */
  uint8_t* x_qT;        /* [K,M] transposed copy, or NULL       */
  uint8_t* w_q;         /* [N,K] e4m3 codes of W                */
  uint8_t* w_qT;        /* [K,N] transposed copy, or NULL       */
  fp8sg_scale_rec* x_sc;
  fp8sg_scale_rec* w_sc;
} fp8_linear_saved;

/* Backward workspace: the quantized gradient and its scale record. */
typedef struct fp8_linear_bwd_ws {
  uint8_t* gy_q;        /* [M,N] e5m2 codes of gy               */
  uint8_t* gy_qT;       /* [N,M] transposed copy, or NULL       */
  fp8sg_scale_rec* gy_sc;
} fp8_linear_bwd_ws;

/*
 * Forward of the FP8 linear layer y = x @ W^T [FP8-TRAIN §4 forward, §6]:
 * amax of x and W, fp64 scales, e4m3 quantize-cast (with the transposed
 * copies `saved` asks for), then the scaled GEMM.
 *   x: [M,K] bf16, w: [N,K] bf16 (nn.Linear's [out,in]); y: [M,N] of type
 *   `out` (FP8SG_OUT_BF16 normally).  M, N, K > 0, multiples of 16.
 * A layer with M*K, N*K and M*N all at most 65536 and no transposed copies
 * runs in one launch (the GEMM blocks reduce and cast what they need); the
 * codes, records and y are the same bits as the separate launches give.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                   int64_t K, const fp8_linear_saved* saved, void* y,
                                   fp8sg_out out, fp8sg_stream stream);

/*
 * Backward of the FP8 linear layer [FP8-TRAIN §4 backward]: gy quantized to
 * e5m2 (with its transposed copy when ws has one), then
 *   dgrad gx[M,K] = gy @ W     from gy_q [M,N] and the saved w_qT [K,N],
 *   wgrad gW[N,K] = gy^T @ x   from gy_qT [N,M] and the saved x_qT [K,M],
 * each dequantised by the product of its two inverse scales (a missing
 * transposed copy is read from the row-major codes, same bits).
 *   gy: [M,N] bf16; gx, gw of type `out` (FP8SG_OUT_F16 feeds fp16 AMP).
 *   `saved` must come from fp8_scaled_linear_fwd with the same M, N, K.
 * Small layers without transposed copies (as for the forward) run the cast
 * of gy and both GEMMs in one launch.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_bwd(const uint16_t* gy, const fp8_linear_saved* saved,
                                   int64_t M, int64_t N, int64_t K, const fp8_linear_bwd_ws* ws,
                                   void* gx, void* gw, fp8sg_out out, fp8sg_stream stream);

/*
 * fp8_scaled_linear_bwd with fp16 gradients and the GradScaler's unscale and
 * non-finite check fused into the two GEMM epilogues [PT-CH20 §20.2.2: unscale
 * the gradients, then check them for inf/NaN; FP8-TRAIN §4 backward].  The
 * results are those of
 *   fp8_scaled_linear_bwd(gy, saved, M, N, K, ws, gx, gw, FP8SG_OUT_F16)
 *   amp_unscale_check({gx, gw}, {M*K, N*K}, 2, scale, found_inf)
 * bit for bit: each element is stored as fp16(fl32(h) * fl32(1.0f / *scale))
 * with h = fp16(acc * alpha), and *found_inf is set to 1 (never cleared) if a
 * stored value is inf or NaN.  The separate pass over gx and gW (4 B per
 * element) is saved.
 *   scale: device float, the current loss scale; found_inf: device int32.
 *   gx: [M,K] fp16, gw: [N,K] fp16 (bit patterns).
 * The other arguments as fp8_scaled_linear_bwd.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_bwd_unscale(const uint16_t* gy,
                                   const fp8_linear_saved* saved, int64_t M, int64_t N, int64_t K,
                                   const fp8_linear_bwd_ws* ws, const float* scale,
                                   int32_t* found_inf, uint16_t* gx, uint16_t* gw,
                                   fp8sg_stream stream);

/*
 * Delayed scaling [PT-CH20 §20.5.9: each FP8 op keeps an amax history of its
 * input and takes every step's scale from the amax of earlier steps].
 * One pass over x instead of fp8_amax + fp8_quantize:
 *   a   = the largest entry of amax_history[0 .. history_len) (NaN if any
 *         entry is NaN, negative entries count as 0)
 *   scale, inv, scale32, inv32 = as fp8_quantize computes them from amax a,
 *         written to rec
 *   q (and qT) = the codes of x at that scale, as fp8_quantize
 *   rec->amax  = max |x| of this x (as fp8_amax), then pushed to the front of
 *         the history: amax_history[i + 1] = old amax_history[i], and
 *         amax_history[0] = rec->amax.
 * Before the first step the caller seeds the history (for example with
 * fp8_amax of the first tensor, or with the amax it expects).
 *   amax_history: device float[history_len], 1 <= history_len <=
 *                 FP8SG_MAX_HISTORY (FP8SG_ERR_SHAPE otherwise), read and
 *                 updated in place, most recent first.
 * The other arguments as fp8_quantize.
 */
FP8SG_API fp8sg_status fp8_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols,
                                  fp8sg_format fmt, float* amax_history, int32_t history_len,
                                  fp8sg_scale_rec* rec, uint8_t* q, uint8_t* qT,
                                  fp8sg_stream stream);

/*
 * fp8_scaled_linear_fwd / fp8_scaled_linear_bwd with delayed scaling of the
 * operands they quantize [PT-CH20 §20.5.9; FP8-TRAIN §4]: x and W (forward,
 * histories hist_x and hist_w) and gy (backward, hist_gy) are cast as
 * fp8_quantize_delayed does, with their histories updated in place; the
 * GEMMs and everything else are as in the dynamic entry points.  The
 * backward reuses the codes and inverse scales the forward saved.
 *   hist_*: device float[history_len], 1 <= history_len <= FP8SG_MAX_HISTORY.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_fwd_delayed(const uint16_t* x, const uint16_t* w,
                                   int64_t M, int64_t N, int64_t K,
                                   const fp8_linear_saved* saved, float* hist_x, float* hist_w,
                                   int32_t history_len, void* y, fp8sg_out out,
                                   fp8sg_stream stream);
FP8SG_API fp8sg_status fp8_scaled_linear_bwd_delayed(const uint16_t* gy, const fp8_linear_saved* saved,
                                   int64_t M, int64_t N, int64_t K, const fp8_linear_bwd_ws* ws,
                                   float* hist_gy, int32_t history_len, void* gx, void* gw,
                                   fp8sg_out out, fp8sg_stream stream);

/*
 * fp8_scaled_linear_bwd_delayed with fp16 gradients and the GradScaler's
 * unscale and non-finite check fused into the GEMM epilogues [PT-CH20 §20.5.9,
 * §20.2.2]: bit for bit
 *   fp8_scaled_linear_bwd_delayed(..., gx, gw, FP8SG_OUT_F16)
 *   amp_unscale_check({gx, gw}, {M*K, N*K}, 2, scale, found_inf)
 * as fp8_scaled_linear_bwd_unscale is for the dynamic backward.
 *   scale: device float; found_inf: device int32 (set, never cleared);
 *   gx: [M,K] fp16, gw: [N,K] fp16.
 * The other arguments as fp8_scaled_linear_bwd_delayed.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_bwd_delayed_unscale(const uint16_t* gy,
                                   const fp8_linear_saved* saved, int64_t M, int64_t N, int64_t K,
                                   const fp8_linear_bwd_ws* ws, float* hist_gy,
                                   int32_t history_len, const float* scale, int32_t* found_inf,
                                   uint16_t* gx, uint16_t* gw, fp8sg_stream stream);

/*
 * Row-wise scaling [FP8-TRAIN §1: instead of one scale per tensor, each row
 * gets its own scale factor, which the accumulation has to carry through].
 * For a rows x cols bf16 matrix x and each row i:
 *   row_amax[i] = max_j |x[i,j]|   (fp32; canonical NaN if the row has a NaN)
 *   s_i = fp8_max / max(row_amax[i], EPS) in fp64, row_inv[i] = 1.0 / s_i
 *   q[i,j] = enc(clamp(fl32(x[i,j] * fl32(s_i)), -max, max))
 * i.e. each row is cast exactly as fp8_quantize casts a one-row tensor.  With
 * qT, the same per column j (col_amax[j], col_inv[j]) and
 *   qT[j,i] = the code of x[i,j] at column j's scale,
 * the row-wise cast of x^T: the operand a GEMM contracting over the rows of x
 * needs (its codes differ from the transpose of q).
 *   x: rows x cols bf16, row-major; rows, cols >= 0 and multiples of 16.
 *   row_amax: device float[rows] (4-byte aligned), row_inv: device
 *   double[rows] (8-byte aligned), both written; q: rows x cols codes.
 *   qT: cols x rows codes; col_amax: float[cols], col_inv: double[cols],
 *   written.  All three NULL skips the transposed cast; otherwise all three
 *   are required (qT may be NULL when rows * cols == 0).
 * Three kernels on `stream`: per-tile partial maxima (kept in q's memory,
 * which the cast then overwrites), their reduction into the vectors, the
 * cast.  An empty dimension leaves the other one's maxima 0 (scale of amax 0).
 */
FP8SG_API fp8sg_status fp8_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                                  fp8sg_format fmt, float* row_amax, double* row_inv,
                                  uint8_t* q, float* col_amax, double* col_inv, uint8_t* qT,
                                  fp8sg_stream stream);

/*
 * Scaled FP8 GEMM with row-wise scales [FP8-TRAIN §1]: as fp8_gemm, with
 * element (m, n) scaled by fl32(inv_a[m] * inv_b[n]):
 *   C[m,n] = out( (sum_k dec(A[m,k]) * dec(B[n,k])) * fl32(inv_a[m] * inv_b[n]) )
 * (each scale is constant along the contraction, so it factors out of the sum).
 *   inv_a: device double[M], inv_b: device double[N], 8-byte aligned.
 * The other arguments as fp8_gemm.
 */
FP8SG_API fp8sg_status fp8_gemm_rowwise(const uint8_t* A, fp8sg_format fa, const uint8_t* B,
                              fp8sg_format fb, const double* inv_a, const double* inv_b,
                              void* C, fp8sg_out out, int64_t M, int64_t N, int64_t Kc,
                              fp8sg_stream stream);

/*
 * What the row-wise forward saves [FP8-TRAIN §1, §6]: codes and scale vectors
 * of x [M,K] and W [N,K], by rows (the forward GEMM) and by columns (the
 * transposed copies the backward GEMMs contract).  Caller-owned device
 * buffers; amax vectors 4-byte, inverse vectors 8-byte, codes 16-byte aligned.
 */
typedef struct fp8_linear_saved_rw {
  uint8_t* x_q;        /* [M,K] codes, one scale per row of x     */
  uint8_t* x_qT;       /* [K,M] codes, one scale per column of x  */
  uint8_t* w_q;        /* [N,K] codes, one scale per row of W     */
  uint8_t* w_qT;       /* [K,N] codes, one scale per column of W  */
  float* x_row_amax;   /* [M] */
  double* x_row_inv;   /* [M] */
  float* x_col_amax;   /* [K] */
  double* x_col_inv;   /* [K] */
  float* w_row_amax;   /* [N] */
  double* w_row_inv;   /* [N] */
  float* w_col_amax;   /* [K] */
  double* w_col_inv;   /* [K] */
} fp8_linear_saved_rw;

/* Row-wise backward workspace: gy [M,N] cast by rows and by columns. */
typedef struct fp8_linear_bwd_ws_rw {
  uint8_t* gy_q;       /* [M,N] e5m2 codes, one scale per row     */
  uint8_t* gy_qT;      /* [N,M] e5m2 codes, one scale per column  */
  float* gy_row_amax;  /* [M] */
  double* gy_row_inv;  /* [M] */
  float* gy_col_amax;  /* [N] */
  double* gy_col_inv;  /* [N] */
} fp8_linear_bwd_ws_rw;

/*
 * The FP8 linear layer with row-wise scaling [FP8-TRAIN §1, §4].
 * Forward: x and W cast as fp8_quantize_rowwise (e4m3, with transposed
 * copies), then y = x_q . w_q^T scaled by x_row_inv[m] * w_row_inv[n].
 * Backward: gy cast the same way in e5m2, then
 *   gx[M,K] = gy_q . w_qT^T     scaled by gy_row_inv[m] * w_col_inv[k]
 *   gW[N,K] = gy_qT . x_qT^T    scaled by gy_col_inv[n] * x_col_inv[k]
 * so every scale lies along a dimension its GEMM does not contract.
 * Shapes, outputs and errors as fp8_scaled_linear_fwd / _bwd; `saved` must
 * come from the row-wise forward with the same M, N, K.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_fwd_rowwise(const uint16_t* x, const uint16_t* w,
                                   int64_t M, int64_t N, int64_t K,
                                   const fp8_linear_saved_rw* saved, void* y, fp8sg_out out,
                                   fp8sg_stream stream);
FP8SG_API fp8sg_status fp8_scaled_linear_bwd_rowwise(const uint16_t* gy,
                                   const fp8_linear_saved_rw* saved, int64_t M, int64_t N,
                                   int64_t K, const fp8_linear_bwd_ws_rw* ws, void* gx, void* gw,
                                   fp8sg_out out, fp8sg_stream stream);

/*
 * fp8_scaled_linear_bwd_rowwise with fp16 gradients and the GradScaler's
 * unscale and non-finite check fused into the GEMM epilogues [FP8-TRAIN §1;
 * PT-CH20 §20.2.2]: each element is stored as
 * fp16(fl32(h) * fl32(1.0f / *scale)) with h = fp16(acc * fl32(inv_a[m] *
 * inv_b[n])), bit for bit
 *   fp8_scaled_linear_bwd_rowwise(..., gx, gw, FP8SG_OUT_F16)
 *   amp_unscale_check({gx, gw}, {M*K, N*K}, 2, scale, found_inf).
 *   scale: device float; found_inf: device int32 (set, never cleared);
 *   gx: [M,K] fp16, gw: [N,K] fp16.
 * The other arguments as fp8_scaled_linear_bwd_rowwise.
 */
FP8SG_API fp8sg_status fp8_scaled_linear_bwd_rowwise_unscale(const uint16_t* gy,
                                   const fp8_linear_saved_rw* saved, int64_t M, int64_t N,
                                   int64_t K, const fp8_linear_bwd_ws_rw* ws, const float* scale,
                                   int32_t* found_inf, uint16_t* gx, uint16_t* gw,
                                   fp8sg_stream stream);

/*
 * GradScaler unscale + non-finite check over a list of fp16 gradients
 * [PT-CH20 §20.2.2: unscale the gradients, then check for inf/NaN;
 *  AMP-NOTES §4 steps 3-4].  In place, for every element:
 *   g <- fp16_RNE( fl32(g) * fl32(1.0f / *scale) )
 * and *found_inf is set to 1 if any stored result is inf or NaN (it is never
 * cleared here: the flag is OR-accumulated over calls).
 *   grads:  HOST array of ntensors device pointers (each 2-byte aligned;
 *           views into one flat gradient buffer are fine).
 *   numel:  HOST array of ntensors element counts (>= 0, any value).
 *   scale:  device float, the current loss scale.
 *   found_inf: device int32.
 * Up to 8192 tensors per call (FP8SG_ERR_SHAPE beyond).
 */
FP8SG_API fp8sg_status amp_unscale_check(uint16_t* const* grads, const int64_t* numel, int32_t ntensors,
                               const float* scale, int32_t* found_inf, fp8sg_stream stream);

/*
 * Workspace for amp_unscale_check_norm: the number of fp32 slots it needs
 * for these element counts: one per block of 8192 elements (blocks counted
 * with room for any 2-byte alignment of each tensor), rounded up to even, plus
 * 512 (256 fp64 partial sums).  Host function, no device work;
 * -1 for invalid arguments (ntensors outside 0..8192, a NULL or negative
 * numel).
 */
FP8SG_API int64_t amp_norm_workspace_len(const int64_t* numel, int32_t ntensors);

/*
 * amp_unscale_check plus the global 2-norm of the unscaled gradients, in the
 * same pass [AMP-NOTES §6 and MP-06 §四: gradient clipping must run after
 * unscale; clip_grad_norm_ takes the 2-norm of all gradient elements
 * together].  Every stored unscaled value g' contributes g'^2 (exact in fp32
 * for fp16 values); the squares are summed in fp32 in a fixed order (8 per
 * 16-byte load, 4 loads per thread, then a fixed tree over each block of 8192
 * elements) into one slot of `workspace` per block; two small kernels add the
 * slots in fp64 in a fixed order.  Results are identical from run to run,
 * within 20 * 2^-24 (relative) of the exact sum of squares.
 *   workspace: device float[workspace_len], 8-byte aligned, caller-owned
 *              scratch of at least amp_norm_workspace_len(numel, ntensors)
 *              slots (FP8SG_ERR_SHAPE if too short); its contents on return
 *              are unspecified.
 *   sumsq_norm: device float[2], written: [0] = sum of squares rounded to
 *              fp32, [1] = its square root (taken in fp64, rounded to fp32).
 *              Both are inf or NaN when a stored value is (found_inf is set).
 * The other arguments and the unscale/check behave as in amp_unscale_check.
 */
FP8SG_API fp8sg_status amp_unscale_check_norm(uint16_t* const* grads, const int64_t* numel,
                                    int32_t ntensors, const float* scale, int32_t* found_inf,
                                    float* workspace, int64_t workspace_len, float* sumsq_norm,
                                    fp8sg_stream stream);

/*
 * amp_unscale_check_norm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight training loops, harnesses that forbid
 * hipMalloc): the same pass and the same results, bit for bit, with the norm's
 * per-block partial sums kept in a fixed scratch array inside the library
 * instead of a caller workspace.  The call allocates nothing.
 *   The scratch holds FP8SG_NOALLOC_NORM_SLOTS fp32 slots (4 MiB, enough for
 *   about 8.5e9 gradient elements); a call whose tensors need more slots than
 *   that (amp_norm_workspace_len) returns FP8SG_ERR_SHAPE before any launch.
 *   Each GPU the library runs this call on holds its own copy of the array
 *   until the process ends; it is located on the device current on the
 *   calling thread, which must be the device of `stream`.
 *   Calls on one GPU share the array: calls that may overlap in time on one
 *   GPU (other streams, other threads) race and must be serialised by the
 *   caller.  Nothing of a previous call's contents is read.
 * The other arguments and the results as amp_unscale_check_norm.
 */
#define FP8SG_NOALLOC_NORM_SLOTS (1LL << 20)
FP8SG_API fp8sg_status amp_unscale_check_norm_noalloc(uint16_t* const* grads, const int64_t* numel,
                                    int32_t ntensors, const float* scale, int32_t* found_inf,
                                    float* sumsq_norm, fp8sg_stream stream);

/*
 * GradScaler.update() [PT-CH20 §20.5.33], on the device:
 *   if *found_inf: *scale *= backoff_factor; *growth_tracker = 0
 *   else: ++*growth_tracker; if it reaches growth_interval:
 *         *scale *= growth_factor; *growth_tracker = 0
 * then *found_inf is reset to 0, ready for the next step's amp_unscale_check
 * (the optimizer's skip decision must read it before this call).
 *   scale: device float; growth_tracker, found_inf: device int32.
 *   growth_interval >= 1 (FP8SG_ERR_SHAPE otherwise).
 */
FP8SG_API fp8sg_status amp_update_scale(float* scale, int32_t* growth_tracker, int32_t* found_inf,
                              float growth_factor, float backoff_factor,
                              int32_t growth_interval, fp8sg_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8SG_H */
