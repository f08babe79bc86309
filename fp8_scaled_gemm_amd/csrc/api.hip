// C-ABI entry points of libfp8sg: argument validation, then kernel launches on
// the caller's stream.  No device allocation and no host synchronisation.
//
// Sources (web pages; cited by title and section):
//   [FP8-TRAIN]  "FP8训练：量化、自动微分、Torchao" (lzwjava.github.io)
//   [PT-CH20]    "第20章 量化与混合精度训练" (yangyitao.com, PyTorch book ch. 20)
#include <stdint.h>

#include "../../include/fp8sg.h"
#include "launch.hpp"

using namespace fp8sg;

static_assert(sizeof(fp8sg_scale_rec) == 32 + 4 * FP8SG_AMAX_PARTS, "scale record layout");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool fmt_ok(int f) { return f == FP8SG_E4M3FN || f == FP8SG_E5M2; }
bool out_ok(int o) { return o == FP8SG_OUT_BF16 || o == FP8SG_OUT_F16 || o == FP8SG_OUT_F32; }
bool dims16(int64_t v) { return v >= 0 && (v % 16) == 0; }
bool dims16_pos(int64_t v) { return v > 0 && (v % 16) == 0; }
fp8sg_status hip_status(hipError_t e) { return e == hipSuccess ? FP8SG_OK : FP8SG_ERR_HIP; }
bool hist_len_ok(int32_t h) { return h >= 1 && h <= FP8SG_MAX_HISTORY; }
bool hist_ok(const float* h) { return h && (reinterpret_cast<uintptr_t>(h) & 3u) == 0; }
hipStream_t S(fp8sg_stream s) { return reinterpret_cast<hipStream_t>(s); }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Size limits: an a x b tensor has at most FP8SG_MAX_ELEMS elements (tested
// without forming an overflowing product); a matrix dimension of a row-wise
// cast or a GEMM is at most FP8SG_MAX_DIM.
bool elems_ok(int64_t a, int64_t b) {
  return a >= 0 && b >= 0 && (a == 0 || b <= FP8SG_MAX_ELEMS / a);
}
bool mat_ok(int64_t r, int64_t c) { return r <= FP8SG_MAX_DIM && c <= FP8SG_MAX_DIM && elems_ok(r, c); }
bool gemm_ok(int64_t M, int64_t N, int64_t K) { return mat_ok(M, K) && mat_ok(N, K) && mat_ok(M, N); }

// A scale-vector pair (amax float[n], inv double[n]) of a row-wise cast.
fp8sg_status check_vec(const float* amax, const double* inv, int64_t n) {
  if (n > 0 && (!amax || !inv)) return FP8SG_ERR_NULL;
  if (!aligned(amax, 4) || !aligned(inv, 8)) return FP8SG_ERR_ALIGN;
  return FP8SG_OK;
}

fp8sg_status check_gemm(const void* A, int fa, const void* B, int fb, const void* ia,
                        const void* ib, const void* C, int out, int64_t M, int64_t N, int64_t K) {
  if (!fmt_ok(fa) || !fmt_ok(fb) || !out_ok(out)) return FP8SG_ERR_FORMAT;
  if (!dims16(M) || !dims16(N) || !dims16(K) || !gemm_ok(M, N, K)) return FP8SG_ERR_SHAPE;
  // zero-sized operands may come with a NULL data pointer
  if ((M * K > 0 && !A) || (N * K > 0 && !B) || (M * N > 0 && !C) || !ia || !ib)
    return FP8SG_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return FP8SG_ERR_ALIGN;
  if (!aligned(ia, 8) || !aligned(ib, 8)) return FP8SG_ERR_ALIGN;
  return FP8SG_OK;
}

// x_qT and w_qT may each be null: the backward GEMM that would read that
// transposed copy reads the row-major codes contraction-major instead.
fp8sg_status check_saved(const fp8_linear_saved* s) {
  if (!s || !s->x_q || !s->w_q || !s->x_sc || !s->w_sc) return FP8SG_ERR_NULL;
  if (!aligned16(s->x_q) || !aligned16(s->x_qT) || !aligned16(s->w_q) || !aligned16(s->w_qT) ||
      !aligned(s->x_sc, 8) || !aligned(s->w_sc, 8))
    return FP8SG_ERR_ALIGN;
  return FP8SG_OK;
}

}  // namespace

extern "C" {

const char* fp8sg_status_string(int status) {
  switch (status) {
    case FP8SG_OK: return "ok";
    case FP8SG_ERR_NULL: return "null pointer argument";
    case FP8SG_ERR_SHAPE: return "invalid size (negative, above the size limits, or not a required multiple of 16)";
    case FP8SG_ERR_ALIGN: return "pointer not aligned (16 bytes for tensors, 8 for records and fp64 vectors, 4 for scalars)";
    case FP8SG_ERR_FORMAT: return "unknown format or output type";
    case FP8SG_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int fp8sg_version(void) { return 100; }

fp8sg_status fp8_linear_copies(int64_t M, int64_t N, int64_t K, int32_t* x_T, int32_t* w_T,
                               int32_t* gy_T) {
  if (!x_T || !w_T || !gy_T) return FP8SG_ERR_NULL;
  if (!dims16_pos(M) || !dims16_pos(N) || !dims16_pos(K) || !gemm_ok(M, N, K))
    return FP8SG_ERR_SHAPE;
  bool x = false, w = false, g = false;
  linear_copies(M, N, K, x, w, g);
  *x_T = x;
  *w_T = w;
  *gy_T = g;
  return FP8SG_OK;
}

fp8sg_status fp8_amax(const uint16_t* x, int64_t n, fp8sg_scale_rec* rec, fp8sg_stream stream) {
  if (!rec || (n > 0 && !x)) return FP8SG_ERR_NULL;
  if (n < 0 || n > FP8SG_MAX_ELEMS) return FP8SG_ERR_SHAPE;
  if (!aligned16(x) || !aligned(rec, 8)) return FP8SG_ERR_ALIGN;
  AmaxArgs a{};
  a.job[0] = AmaxJob{x, n, rec, 0, amax_blocks_for(n)};
  a.njobs = 1;
  return hip_status(launch_amax(a, true, S(stream)));
}

fp8sg_status fp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, fp8sg_format fmt,
                          fp8sg_scale_rec* rec, uint8_t* q, uint8_t* qT, fp8sg_stream stream) {
  if (!rec) return FP8SG_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8SG_ERR_FORMAT;
  if (!elems_ok(rows, cols)) return FP8SG_ERR_SHAPE;
  if (rows * cols > 0 && (!x || !q)) return FP8SG_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (qT && !aligned16(qT)) || !aligned(rec, 8))
    return FP8SG_ERR_ALIGN;
  QuantArgs a{};
  a.job[0] = QuantJob{x, rows, cols, rec, q, qT, 0, 0, 0};
  a.njobs = 1;
  return hip_status(launch_quantize(a, fmt, S(stream)));
}

fp8sg_status fp8_amax_f16(const uint16_t* x, int64_t n, fp8sg_scale_rec* rec, fp8sg_stream stream) {
  if (!rec || (n > 0 && !x)) return FP8SG_ERR_NULL;
  if (n < 0 || n > FP8SG_MAX_ELEMS) return FP8SG_ERR_SHAPE;
  if (!aligned16(x) || !aligned(rec, 8)) return FP8SG_ERR_ALIGN;
  AmaxArgs a{};
  a.job[0] = AmaxJob{x, n, rec, 0, amax_blocks_for(n)};
  a.njobs = 1;
  a.in_f16 = 1;
  return hip_status(launch_amax(a, true, S(stream)));
}

fp8sg_status fp8_quantize_f16(const uint16_t* x, int64_t rows, int64_t cols, fp8sg_format fmt,
                              fp8sg_scale_rec* rec, uint8_t* q, uint8_t* qT, fp8sg_stream stream) {
  if (!rec) return FP8SG_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8SG_ERR_FORMAT;
  if (!elems_ok(rows, cols)) return FP8SG_ERR_SHAPE;
  if (rows * cols > 0 && (!x || !q)) return FP8SG_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (qT && !aligned16(qT)) || !aligned(rec, 8))
    return FP8SG_ERR_ALIGN;
  QuantArgs a{};
  a.job[0] = QuantJob{x, rows, cols, rec, q, qT, 0, 0, 0};
  a.njobs = 1;
  a.in_f16 = 1;
  return hip_status(launch_quantize(a, fmt, S(stream)));
}

fp8sg_status fp8_quantize_from_amax(const uint16_t* x, int64_t rows, int64_t cols,
                                    fp8sg_format fmt, const float* amax, fp8sg_scale_rec* rec,
                                    uint8_t* q, uint8_t* qT, fp8sg_stream stream) {
  if (!rec || !amax) return FP8SG_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8SG_ERR_FORMAT;
  if (!elems_ok(rows, cols)) return FP8SG_ERR_SHAPE;
  if (rows * cols > 0 && (!x || !q)) return FP8SG_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (qT && !aligned16(qT)) || !aligned(rec, 8) ||
      !aligned(amax, 4))
    return FP8SG_ERR_ALIGN;
  QuantArgs a{};
  a.job[0] = QuantJob{x, rows, cols, rec, q, qT, 0, 0, 0, nullptr, 0, amax};
  a.njobs = 1;
  return hip_status(launch_quantize(a, fmt, S(stream)));
}

fp8sg_status fp8_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols,
                                  fp8sg_format fmt, float* amax_history, int32_t history_len,
                                  fp8sg_scale_rec* rec, uint8_t* q, uint8_t* qT,
                                  fp8sg_stream stream) {
  if (!rec || !amax_history) return FP8SG_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8SG_ERR_FORMAT;
  if (!elems_ok(rows, cols) || !hist_len_ok(history_len)) return FP8SG_ERR_SHAPE;
  if (rows * cols > 0 && (!x || !q)) return FP8SG_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (qT && !aligned16(qT)) || !aligned(rec, 8))
    return FP8SG_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(amax_history) & 3u) return FP8SG_ERR_ALIGN;
  QuantArgs a{};
  a.job[0] = QuantJob{x, rows, cols, rec, q, qT, 0, 0, 0, amax_history, history_len};
  a.njobs = 1;
  return hip_status(launch_quantize(a, fmt, S(stream)));
}

fp8sg_status fp8_gemm(const uint8_t* A, fp8sg_format fa, const uint8_t* B, fp8sg_format fb,
                      const double* inv_a, const double* inv_b, void* C, fp8sg_out out,
                      int64_t M, int64_t N, int64_t Kc, fp8sg_stream stream) {
  fp8sg_status st = check_gemm(A, fa, B, fb, inv_a, inv_b, C, out, M, N, Kc);
  if (st != FP8SG_OK) return st;
  GemmProblem p{A, B, C, inv_a, inv_b, M, N, Kc};
  return hip_status(launch_gemm(p, fa, fb, out, S(stream)));
}

fp8sg_status fp8_gemm_kmajor(const uint8_t* A, fp8sg_format fa, int32_t a_kmajor, const uint8_t* B,
                             fp8sg_format fb, int32_t b_kmajor, const double* inv_a,
                             const double* inv_b, void* C, fp8sg_out out, int64_t M, int64_t N,
                             int64_t Kc, fp8sg_stream stream) {
  fp8sg_status st = check_gemm(A, fa, B, fb, inv_a, inv_b, C, out, M, N, Kc);
  if (st != FP8SG_OK) return st;
  GemmProblem p{A, B, C, inv_a, inv_b, M, N, Kc};
  return hip_status(launch_gemm_km(p, fa, fb, out, a_kmajor != 0, b_kmajor != 0, S(stream)));
}

fp8sg_status fp8_gemm_kmajor_unscale(const uint8_t* A, fp8sg_format fa, int32_t a_kmajor,
                                     const uint8_t* B, fp8sg_format fb, int32_t b_kmajor,
                                     const double* inv_a, const double* inv_b,
                                     const float* amp_scale, int32_t* found_inf, uint16_t* C,
                                     int64_t M, int64_t N, int64_t Kc, fp8sg_stream stream) {
  fp8sg_status st = check_gemm(A, fa, B, fb, inv_a, inv_b, C, FP8SG_OUT_F16, M, N, Kc);
  if (st != FP8SG_OK) return st;
  if (!amp_scale || !found_inf) return FP8SG_ERR_NULL;
  if (!aligned(amp_scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  GemmProblem p{A, B, C, inv_a, inv_b, M, N, Kc, amp_scale, found_inf};
  return hip_status(launch_gemm_km(p, fa, fb, kOutF16Unscale, a_kmajor != 0, b_kmajor != 0, S(stream)));
}

fp8sg_status fp8_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, fp8sg_format fmt,
                                  float* row_amax, double* row_inv, uint8_t* q, float* col_amax,
                                  double* col_inv, uint8_t* qT, fp8sg_stream stream) {
  if (!fmt_ok(fmt)) return FP8SG_ERR_FORMAT;
  if (!dims16(rows) || !dims16(cols) || !mat_ok(rows, cols)) return FP8SG_ERR_SHAPE;
  if (rows * cols > 0 && (!x || !q)) return FP8SG_ERR_NULL;
  fp8sg_status st = check_vec(row_amax, row_inv, rows);
  if (st != FP8SG_OK) return st;
  const bool with_t = col_amax || col_inv || qT;
  if (with_t) {
    st = check_vec(col_amax, col_inv, cols);
    if (st != FP8SG_OK) return st;
    if (rows * cols > 0 && !qT) return FP8SG_ERR_NULL;
  }
  if (!aligned16(x) || !aligned16(q) || !aligned16(qT)) return FP8SG_ERR_ALIGN;
  RowwiseArgs a{x, rows, cols, row_amax, row_inv, q, col_amax, col_inv, qT, 0};
  return hip_status(launch_rowwise(a, fmt, S(stream)));
}

fp8sg_status fp8_gemm_rowwise(const uint8_t* A, fp8sg_format fa, const uint8_t* B, fp8sg_format fb,
                              const double* inv_a, const double* inv_b, void* C, fp8sg_out out,
                              int64_t M, int64_t N, int64_t Kc, fp8sg_stream stream) {
  fp8sg_status st = check_gemm(A, fa, B, fb, inv_a, inv_b, C, out, M, N, Kc);
  if (st != FP8SG_OK) return st;
  GemmProblem p{A, B, C, inv_a, inv_b, M, N, Kc};
  return hip_status(launch_gemm_rowwise(p, fa, fb, out, S(stream)));
}

fp8sg_status fp8_gemm_unscale(const uint8_t* A, fp8sg_format fa, const uint8_t* B, fp8sg_format fb,
                              const double* inv_a, const double* inv_b, const float* scale,
                              int32_t* found_inf, uint16_t* C, int64_t M, int64_t N, int64_t Kc,
                              fp8sg_stream stream) {
  fp8sg_status st = check_gemm(A, fa, B, fb, inv_a, inv_b, C, FP8SG_OUT_F16, M, N, Kc);
  if (st != FP8SG_OK) return st;
  if (!scale || !found_inf) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  GemmProblem p{A, B, C, inv_a, inv_b, M, N, Kc, scale, found_inf};
  return hip_status(launch_gemm_unscale(p, fa, fb, S(stream)));
}

}  // extern "C"

namespace {

fp8sg_status check_saved_rw(const fp8_linear_saved_rw* s, int64_t M, int64_t N, int64_t K) {
  if (!s || !s->x_q || !s->x_qT || !s->w_q || !s->w_qT) return FP8SG_ERR_NULL;
  if (!aligned16(s->x_q) || !aligned16(s->x_qT) || !aligned16(s->w_q) || !aligned16(s->w_qT))
    return FP8SG_ERR_ALIGN;
  const fp8sg_status sts[4] = {check_vec(s->x_row_amax, s->x_row_inv, M),
                               check_vec(s->x_col_amax, s->x_col_inv, K),
                               check_vec(s->w_row_amax, s->w_row_inv, N),
                               check_vec(s->w_col_amax, s->w_col_inv, K)};
  for (fp8sg_status st : sts)
    if (st != FP8SG_OK) return st;
  return FP8SG_OK;
}

// Forward [FP8-TRAIN §4 forward, §6]: codes and transposed copies of x and W
// (dynamic: one amax launch over both, then one quantize launch; delayed: one
// quantize launch that also reduces the current amax, then the history push),
// then one GEMM.
fp8sg_status linear_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                        const fp8_linear_saved* saved, float* hist_x, float* hist_w,
                        int32_t hist_len, void* y, fp8sg_out out, fp8sg_stream stream) {
  if (!x || !w || !y) return FP8SG_ERR_NULL;
  fp8sg_status st = check_saved(saved);
  if (st != FP8SG_OK) return st;
  if (!out_ok(out)) return FP8SG_ERR_FORMAT;
  if (!dims16_pos(M) || !dims16_pos(N) || !dims16_pos(K) || !gemm_ok(M, N, K))
    return FP8SG_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return FP8SG_ERR_ALIGN;
  const bool delayed = hist_x || hist_w;
  if (delayed) {
    if (!hist_x || !hist_w) return FP8SG_ERR_NULL;
    if (!hist_len_ok(hist_len)) return FP8SG_ERR_SHAPE;
    if (!hist_ok(hist_x) || !hist_ok(hist_w)) return FP8SG_ERR_ALIGN;
  }
  hipStream_t s = S(stream);
  hipError_t e;
  if (!delayed && !saved->x_qT && !saved->w_qT && small_layer_fits(M, N, K)) {
    // small layer without transposed copies: casts and GEMM in one launch
    SmallFwdArgs a{x, w, GemmProblem{saved->x_q, saved->w_q, y, nullptr, nullptr, M, N, K},
                   saved->x_sc, saved->w_sc, saved->x_q, saved->w_q};
    return hip_status(launch_small_fwd(a, out, s));
  }
  QuantArgs qa{};
  qa.job[0] = QuantJob{x, M, K, saved->x_sc, saved->x_q, saved->x_qT, 0, 0, 0, hist_x, hist_len};
  qa.job[1] = QuantJob{w, N, K, saved->w_sc, saved->w_q, saved->w_qT, 0, 0, 0, hist_w, hist_len};
  qa.njobs = 2;
  if (!delayed && self_cast_fits(qa)) {  // small x and W: amax and cast in one launch
    e = launch_quantize_self(qa, FP8SG_E4M3FN, s);
  } else {
    if (!delayed) {
      AmaxArgs am{};
      am.job[0] = AmaxJob{x, M * K, saved->x_sc, 0, amax_blocks_for(M * K)};
      am.job[1] = AmaxJob{w, N * K, saved->w_sc, 0, amax_blocks_for(N * K)};
      am.njobs = 2;
      e = launch_amax(am, false, s);
      if (e != hipSuccess) return FP8SG_ERR_HIP;
    }
    e = launch_quantize(qa, FP8SG_E4M3FN, s);
  }
  if (e != hipSuccess) return FP8SG_ERR_HIP;

  GemmProblem p{saved->x_q, saved->w_q, y, &saved->x_sc->inv, &saved->w_sc->inv, M, N, K};
  return hip_status(launch_gemm(p, FP8SG_E4M3FN, FP8SG_E4M3FN, out, s));
}

// Backward [FP8-TRAIN §4 backward]: gy -> e5m2 codes + transposed copy, then
// dgrad (gy_q [M,N] x w_qT [K,N]^T) and wgrad (gy_qT [N,M] x x_qT [K,M]^T).
fp8sg_status linear_bwd(const uint16_t* gy, const fp8_linear_saved* saved, int64_t M, int64_t N,
                        int64_t K, const fp8_linear_bwd_ws* ws, float* hist_gy, int32_t hist_len,
                        void* gx, void* gw, fp8sg_out out, fp8sg_stream stream,
                        const float* amp_scale = nullptr, int32_t* found_inf = nullptr) {
  if (!gy || !ws || !gx || !gw) return FP8SG_ERR_NULL;
  fp8sg_status st = check_saved(saved);
  if (st != FP8SG_OK) return st;
  if (!ws->gy_q || !ws->gy_sc) return FP8SG_ERR_NULL;
  if (!out_ok(out)) return FP8SG_ERR_FORMAT;
  if (!dims16_pos(M) || !dims16_pos(N) || !dims16_pos(K) || !gemm_ok(M, N, K))
    return FP8SG_ERR_SHAPE;
  if (!aligned16(gy) || !aligned16(gx) || !aligned16(gw) || !aligned16(ws->gy_q) ||
      !aligned16(ws->gy_qT) || !aligned(ws->gy_sc, 8))
    return FP8SG_ERR_ALIGN;
  if (hist_gy) {
    if (!hist_len_ok(hist_len)) return FP8SG_ERR_SHAPE;
    if (!hist_ok(hist_gy)) return FP8SG_ERR_ALIGN;
  }
  hipStream_t s = S(stream);
  hipError_t e;
  // An operand without its transposed copy is read from its row-major codes,
  // contraction-major: dgrad's W codes [N, K] as B^T, wgrad's gy codes
  // [M, N] as A^T and x codes [M, K] as B^T.
  const bool tb_d = !saved->w_qT, ta_w = !ws->gy_qT, tb_w = !saved->x_qT;
  const int o = amp_scale ? kOutF16Unscale : (int)out;
  if (!hist_gy && tb_d && ta_w && tb_w && small_layer_fits(M, N, K)) {
    // small layer without transposed copies: the cast of gy and both GEMMs
    // in one launch
    SmallBwdArgs a{gy, M, N,
                   GemmProblem{ws->gy_q, saved->w_q, gx, nullptr, &saved->w_sc->inv, M, K, N,
                               amp_scale, found_inf},
                   GemmProblem{ws->gy_q, saved->x_q, gw, nullptr, &saved->x_sc->inv, N, K, M,
                               amp_scale, found_inf},
                   ws->gy_sc, ws->gy_q};
    return hip_status(launch_small_bwd(a, o, s));
  }
  QuantArgs qa{};
  qa.job[0] = QuantJob{gy, M, N, ws->gy_sc, ws->gy_q, ws->gy_qT, 0, 0, 0, hist_gy, hist_len};
  qa.njobs = 1;
  if (!hist_gy && self_cast_fits(qa)) {  // small gy: amax and cast in one launch
    e = launch_quantize_self(qa, FP8SG_E5M2, s);
  } else {
    if (!hist_gy) {
      AmaxArgs am{};
      am.job[0] = AmaxJob{gy, M * N, ws->gy_sc, 0, amax_blocks_for(M * N)};
      am.njobs = 1;
      e = launch_amax(am, false, s);
      if (e != hipSuccess) return FP8SG_ERR_HIP;
    }
    e = launch_quantize(qa, FP8SG_E5M2, s);
  }
  if (e != hipSuccess) return FP8SG_ERR_HIP;

  GemmProblem dg{ws->gy_q, tb_d ? saved->w_q : saved->w_qT, gx, &ws->gy_sc->inv, &saved->w_sc->inv,
                 M, K, N, amp_scale, found_inf};
  GemmProblem wg{ta_w ? ws->gy_q : ws->gy_qT, tb_w ? saved->x_q : saved->x_qT, gw, &ws->gy_sc->inv,
                 &saved->x_sc->inv, N, K, M, amp_scale, found_inf};
  if (tb_d && ta_w && tb_w) return hip_status(launch_gemm_km_pair(dg, wg, o, s));
  if (tb_d || ta_w || tb_w) {  // some copies kept: one launch per GEMM
    e = launch_gemm_km(dg, FP8SG_E5M2, FP8SG_E4M3FN, o, false, tb_d, s);
    if (e != hipSuccess) return FP8SG_ERR_HIP;
    return hip_status(launch_gemm_km(wg, FP8SG_E5M2, FP8SG_E4M3FN, o, ta_w, tb_w, s));
  }
  if (amp_scale)  // fp16 gradients unscaled and checked in the GEMM epilogues
    return hip_status(launch_gemm_unscale_pair(dg, wg, false, s));
  return hip_status(launch_gemm_pair(dg, wg, FP8SG_E5M2, FP8SG_E4M3FN, out, s));
}

// Row-wise backward [FP8-TRAIN §1, §4 backward]: gy cast by rows and by
// columns (e5m2); dgrad from gy_q (rows of gy) and w_qT (columns of W), wgrad
// from gy_qT (columns of gy) and x_qT (columns of x): every scale lies along a
// dimension the GEMM does not contract.  With amp_scale the fp16 gradients are
// unscaled and checked in the GEMM epilogues.
fp8sg_status linear_bwd_rw(const uint16_t* gy, const fp8_linear_saved_rw* saved, int64_t M,
                                  int64_t N, int64_t K, const fp8_linear_bwd_ws_rw* ws, void* gx,
                                  void* gw, fp8sg_out out, fp8sg_stream stream,
                                  const float* amp_scale = nullptr, int32_t* found_inf = nullptr) {
  if (!gy || !ws || !gx || !gw) return FP8SG_ERR_NULL;
  if (!out_ok(out)) return FP8SG_ERR_FORMAT;
  if (!dims16_pos(M) || !dims16_pos(N) || !dims16_pos(K) || !gemm_ok(M, N, K))
    return FP8SG_ERR_SHAPE;
  fp8sg_status st = check_saved_rw(saved, M, N, K);
  if (st != FP8SG_OK) return st;
  if (!ws->gy_q || !ws->gy_qT) return FP8SG_ERR_NULL;
  st = check_vec(ws->gy_row_amax, ws->gy_row_inv, M);
  if (st != FP8SG_OK) return st;
  st = check_vec(ws->gy_col_amax, ws->gy_col_inv, N);
  if (st != FP8SG_OK) return st;
  if (!aligned16(gy) || !aligned16(gx) || !aligned16(gw) || !aligned16(ws->gy_q) ||
      !aligned16(ws->gy_qT))
    return FP8SG_ERR_ALIGN;
  hipStream_t s = S(stream);
  const fp8_linear_saved_rw& v = *saved;
  RowwiseArgs ag{gy, M, N, ws->gy_row_amax, ws->gy_row_inv, ws->gy_q, ws->gy_col_amax,
                 ws->gy_col_inv, ws->gy_qT, 0};
  if (launch_rowwise(ag, FP8SG_E5M2, s) != hipSuccess) return FP8SG_ERR_HIP;
  GemmProblem dg{ws->gy_q, v.w_qT, gx, ws->gy_row_inv, v.w_col_inv, M, K, N, amp_scale, found_inf};
  GemmProblem wg{ws->gy_qT, v.x_qT, gw, ws->gy_col_inv, v.x_col_inv, N, K, M, amp_scale, found_inf};
  if (amp_scale) return hip_status(launch_gemm_unscale_pair(dg, wg, true, s));
  return hip_status(launch_gemm_rowwise_pair(dg, wg, out, s));
}

}  // namespace

extern "C" {

fp8sg_status fp8_scaled_linear_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                   int64_t K, const fp8_linear_saved* saved, void* y,
                                   fp8sg_out out, fp8sg_stream stream) {
  return linear_fwd(x, w, M, N, K, saved, nullptr, nullptr, 0, y, out, stream);
}

fp8sg_status fp8_scaled_linear_fwd_delayed(const uint16_t* x, const uint16_t* w, int64_t M,
                                           int64_t N, int64_t K, const fp8_linear_saved* saved,
                                           float* hist_x, float* hist_w, int32_t history_len,
                                           void* y, fp8sg_out out, fp8sg_stream stream) {
  if (!hist_x || !hist_w) return FP8SG_ERR_NULL;
  return linear_fwd(x, w, M, N, K, saved, hist_x, hist_w, history_len, y, out, stream);
}

fp8sg_status fp8_scaled_linear_bwd(const uint16_t* gy, const fp8_linear_saved* saved,
                                   int64_t M, int64_t N, int64_t K, const fp8_linear_bwd_ws* ws,
                                   void* gx, void* gw, fp8sg_out out, fp8sg_stream stream) {
  return linear_bwd(gy, saved, M, N, K, ws, nullptr, 0, gx, gw, out, stream);
}

fp8sg_status fp8_scaled_linear_bwd_unscale(const uint16_t* gy, const fp8_linear_saved* saved,
                                           int64_t M, int64_t N, int64_t K,
                                           const fp8_linear_bwd_ws* ws, const float* scale,
                                           int32_t* found_inf, uint16_t* gx, uint16_t* gw,
                                           fp8sg_stream stream) {
  if (!scale || !found_inf) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  return linear_bwd(gy, saved, M, N, K, ws, nullptr, 0, gx, gw, FP8SG_OUT_F16, stream, scale,
                    found_inf);
}

fp8sg_status fp8_scaled_linear_bwd_delayed(const uint16_t* gy, const fp8_linear_saved* saved,
                                           int64_t M, int64_t N, int64_t K,
                                           const fp8_linear_bwd_ws* ws, float* hist_gy,
                                           int32_t history_len, void* gx, void* gw,
                                           fp8sg_out out, fp8sg_stream stream) {
  if (!hist_gy) return FP8SG_ERR_NULL;
  return linear_bwd(gy, saved, M, N, K, ws, hist_gy, history_len, gx, gw, out, stream);
}

fp8sg_status fp8_scaled_linear_bwd_delayed_unscale(const uint16_t* gy,
                                                   const fp8_linear_saved* saved, int64_t M,
                                                   int64_t N, int64_t K,
                                                   const fp8_linear_bwd_ws* ws, float* hist_gy,
                                                   int32_t history_len, const float* scale,
                                                   int32_t* found_inf, uint16_t* gx, uint16_t* gw,
                                                   fp8sg_stream stream) {
  if (!hist_gy || !scale || !found_inf) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  return linear_bwd(gy, saved, M, N, K, ws, hist_gy, history_len, gx, gw, FP8SG_OUT_F16, stream,
                    scale, found_inf);
}

// Row-wise forward [FP8-TRAIN §1, §4 forward]: x and W cast with one scale per
// row (codes for this GEMM) and one per column (transposed copies for the
// backward GEMMs), then y = x_q . w_q^T scaled by x_row_inv[m] * w_row_inv[n].
fp8sg_status fp8_scaled_linear_fwd_rowwise(const uint16_t* x, const uint16_t* w, int64_t M,
                                           int64_t N, int64_t K, const fp8_linear_saved_rw* saved,
                                           void* y, fp8sg_out out, fp8sg_stream stream) {
  if (!x || !w || !y) return FP8SG_ERR_NULL;
  if (!out_ok(out)) return FP8SG_ERR_FORMAT;
  if (!dims16_pos(M) || !dims16_pos(N) || !dims16_pos(K) || !gemm_ok(M, N, K))
    return FP8SG_ERR_SHAPE;
  fp8sg_status st = check_saved_rw(saved, M, N, K);
  if (st != FP8SG_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return FP8SG_ERR_ALIGN;
  hipStream_t s = S(stream);
  const fp8_linear_saved_rw& v = *saved;
  RowwiseArgs ax{x, M, K, v.x_row_amax, v.x_row_inv, v.x_q, v.x_col_amax, v.x_col_inv, v.x_qT, 0};
  RowwiseArgs aw{w, N, K, v.w_row_amax, v.w_row_inv, v.w_q, v.w_col_amax, v.w_col_inv, v.w_qT, 0};
  if (launch_rowwise2(ax, aw, FP8SG_E4M3FN, s) != hipSuccess) return FP8SG_ERR_HIP;
  GemmProblem p{v.x_q, v.w_q, y, v.x_row_inv, v.w_row_inv, M, N, K};
  return hip_status(launch_gemm_rowwise(p, FP8SG_E4M3FN, FP8SG_E4M3FN, out, s));
}

fp8sg_status fp8_scaled_linear_bwd_rowwise(const uint16_t* gy, const fp8_linear_saved_rw* saved,
                                           int64_t M, int64_t N, int64_t K,
                                           const fp8_linear_bwd_ws_rw* ws, void* gx, void* gw,
                                           fp8sg_out out, fp8sg_stream stream) {
  return linear_bwd_rw(gy, saved, M, N, K, ws, gx, gw, out, stream);
}

fp8sg_status fp8_scaled_linear_bwd_rowwise_unscale(const uint16_t* gy,
                                                   const fp8_linear_saved_rw* saved, int64_t M,
                                                   int64_t N, int64_t K,
                                                   const fp8_linear_bwd_ws_rw* ws,
                                                   const float* scale, int32_t* found_inf,
                                                   uint16_t* gx, uint16_t* gw,
                                                   fp8sg_stream stream) {
  if (!scale || !found_inf) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  return linear_bwd_rw(gy, saved, M, N, K, ws, gx, gw, FP8SG_OUT_F16, stream, scale, found_inf);
}

fp8sg_status amp_unscale_check(uint16_t* const* grads, const int64_t* numel, int32_t ntensors,
                               const float* scale, int32_t* found_inf, fp8sg_stream stream) {
  if (!scale || !found_inf) return FP8SG_ERR_NULL;
  if (ntensors < 0 || ntensors > 8192) return FP8SG_ERR_SHAPE;
  if (ntensors > 0 && (!grads || !numel)) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  for (int32_t i = 0; i < ntensors; ++i) {
    if (numel[i] < 0 || numel[i] > FP8SG_MAX_ELEMS) return FP8SG_ERR_SHAPE;
    if (numel[i] > 0 && !grads[i]) return FP8SG_ERR_NULL;
    if (numel[i] > 0 && (reinterpret_cast<uintptr_t>(grads[i]) & 1u)) return FP8SG_ERR_ALIGN;
  }
  return hip_status(
      launch_unscale_check(grads, numel, ntensors, scale, found_inf, nullptr, nullptr, S(stream)));
}

int64_t amp_norm_workspace_len(const int64_t* numel, int32_t ntensors) {
  if (ntensors < 0 || ntensors > 8192 || (ntensors > 0 && !numel)) return -1;
  for (int32_t i = 0; i < ntensors; ++i)
    if (numel[i] < 0 || numel[i] > FP8SG_MAX_ELEMS) return -1;
  return unscale_blocks_bound(numel, ntensors);
}

fp8sg_status amp_unscale_check_norm(uint16_t* const* grads, const int64_t* numel,
                                    int32_t ntensors, const float* scale, int32_t* found_inf,
                                    float* workspace, int64_t workspace_len, float* sumsq_norm,
                                    fp8sg_stream stream) {
  if (!scale || !found_inf || !sumsq_norm) return FP8SG_ERR_NULL;
  if (ntensors < 0 || ntensors > 8192) return FP8SG_ERR_SHAPE;
  if (ntensors > 0 && (!grads || !numel)) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  for (int32_t i = 0; i < ntensors; ++i) {
    if (numel[i] < 0 || numel[i] > FP8SG_MAX_ELEMS) return FP8SG_ERR_SHAPE;
    if (numel[i] > 0 && !grads[i]) return FP8SG_ERR_NULL;
    if (numel[i] > 0 && (reinterpret_cast<uintptr_t>(grads[i]) & 1u)) return FP8SG_ERR_ALIGN;
  }
  const int64_t need = norm_slots(grads, numel, ntensors);
  if (workspace_len < need) return FP8SG_ERR_SHAPE;
  if (!workspace) return FP8SG_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(sumsq_norm) & 3u) return FP8SG_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(workspace) & 7u) return FP8SG_ERR_ALIGN;
  return hip_status(launch_unscale_check(grads, numel, ntensors, scale, found_inf, workspace,
                                         sumsq_norm, S(stream)));
}

fp8sg_status amp_unscale_check_norm_noalloc(uint16_t* const* grads, const int64_t* numel,
                                            int32_t ntensors, const float* scale,
                                            int32_t* found_inf, float* sumsq_norm,
                                            fp8sg_stream stream) {
  if (!scale || !found_inf || !sumsq_norm) return FP8SG_ERR_NULL;
  if (ntensors < 0 || ntensors > 8192) return FP8SG_ERR_SHAPE;
  if (ntensors > 0 && (!grads || !numel)) return FP8SG_ERR_NULL;
  if (!aligned(scale, 4) || !aligned(found_inf, 4)) return FP8SG_ERR_ALIGN;
  for (int32_t i = 0; i < ntensors; ++i) {
    if (numel[i] < 0 || numel[i] > FP8SG_MAX_ELEMS) return FP8SG_ERR_SHAPE;
    if (numel[i] > 0 && !grads[i]) return FP8SG_ERR_NULL;
    if (numel[i] > 0 && (reinterpret_cast<uintptr_t>(grads[i]) & 1u)) return FP8SG_ERR_ALIGN;
  }
  if (norm_slots(grads, numel, ntensors) > kNoAllocNormSlots) return FP8SG_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(sumsq_norm) & 3u) return FP8SG_ERR_ALIGN;
  float* ws = nullptr;
  const hipError_t e = norm_scratch(&ws);
  if (e != hipSuccess) return FP8SG_ERR_HIP;
  return hip_status(launch_unscale_check(grads, numel, ntensors, scale, found_inf, ws,
                                         sumsq_norm, S(stream)));
}

fp8sg_status amp_update_scale(float* scale, int32_t* growth_tracker, int32_t* found_inf,
                              float growth_factor, float backoff_factor,
                              int32_t growth_interval, fp8sg_stream stream) {
  if (!scale || !growth_tracker || !found_inf) return FP8SG_ERR_NULL;
  if (growth_interval < 1) return FP8SG_ERR_SHAPE;
  if (!aligned(scale, 4) || !aligned(growth_tracker, 4) || !aligned(found_inf, 4))
    return FP8SG_ERR_ALIGN;
  return hip_status(launch_update_scale(scale, growth_tracker, found_inf, growth_factor,
                                        backoff_factor, growth_interval, S(stream)));
}

}  // extern "C"
