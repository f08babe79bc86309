"""Python binding of libfp8sg, the MI355X (gfx950) FP8 scaled linear layer
(per-tensor dynamic or delayed scaling, or row-wise scaling) and GradScaler
step.

Argument marshalling only: every function forwards torch device tensors as raw
pointers and sizes to the C ABI declared in include/fp8sg.h (same names, same
order), on the current torch stream.  All arithmetic runs in the library's HIP
kernels; torch provides device memory and streams.  There is no fallback: if
the library is not built, importing it raises.
"""
import ctypes
import os

import torch  # loads the HIP runtime the library binds to (one runtime per process)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8sg.so")

E4M3FN, E5M2 = 0, 1
OUT_BF16, OUT_F16, OUT_F32 = 0, 1, 2
AMAX_PARTS = 1024
SCALE_REC_BYTES = 32 + 4 * AMAX_PARTS

EXPORTS = ("fp8sg_status_string", "fp8sg_version", "amp_norm_workspace_len", "fp8_amax",
           "fp8_quantize", "fp8_quantize_delayed", "fp8_gemm", "fp8_scaled_linear_fwd",
           "fp8_scaled_linear_fwd_delayed", "fp8_scaled_linear_bwd", "fp8_scaled_linear_bwd_delayed",
           "amp_unscale_check", "amp_unscale_check_norm", "amp_update_scale",
           "fp8_quantize_rowwise", "fp8_gemm_rowwise", "fp8_scaled_linear_fwd_rowwise",
           "fp8_scaled_linear_bwd_rowwise", "fp8_scaled_linear_bwd_unscale", "fp8_gemm_unscale",
           "fp8_scaled_linear_bwd_delayed_unscale", "fp8_scaled_linear_bwd_rowwise_unscale",
           "fp8_quantize_from_amax", "amp_unscale_check_norm_noalloc", "fp8_amax_f16",
           "fp8_quantize_f16", "fp8_gemm_kmajor", "fp8_gemm_kmajor_unscale", "fp8_linear_copies")
MAX_HISTORY = 1024
MAX_DIM = 1 << 29     # largest matrix dimension an entry point takes
MAX_ELEMS = 1 << 35   # largest tensor, in elements


class Fp8sgError(RuntimeError):
    pass


class _Saved(ctypes.Structure):
    _fields_ = [("x_q", ctypes.c_void_p), ("x_qT", ctypes.c_void_p), ("w_q", ctypes.c_void_p),
                ("w_qT", ctypes.c_void_p), ("x_sc", ctypes.c_void_p), ("w_sc", ctypes.c_void_p)]


class _BwdWs(ctypes.Structure):
    _fields_ = [("gy_q", ctypes.c_void_p), ("gy_qT", ctypes.c_void_p), ("gy_sc", ctypes.c_void_p)]


class _SavedRW(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x_q", "x_qT", "w_q", "w_qT", "x_row_amax", "x_row_inv", "x_col_amax", "x_col_inv",
        "w_row_amax", "w_row_inv", "w_col_amax", "w_col_inv")]


class _BwdWsRW(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "gy_q", "gy_qT", "gy_row_amax", "gy_row_inv", "gy_col_amax", "gy_col_inv")]


_lib = None


def lib():
    """The loaded libfp8sg.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(or python fp8_scaled_gemm_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, f32, i = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                           ctypes.c_int)
    L.fp8sg_status_string.argtypes = [i]
    L.fp8sg_status_string.restype = ctypes.c_char_p
    L.fp8sg_version.restype = i
    L.fp8_amax.argtypes = [P, i64, P, P]
    L.fp8_quantize.argtypes = [P, i64, i64, i, P, P, P, P]
    L.fp8_quantize_delayed.argtypes = [P, i64, i64, i, P, i32, P, P, P, P]
    L.fp8_quantize_from_amax.argtypes = [P, i64, i64, i, P, P, P, P, P]
    L.fp8_amax_f16.argtypes = [P, i64, P, P]
    L.fp8_quantize_f16.argtypes = [P, i64, i64, i, P, P, P, P]
    L.fp8_gemm.argtypes = [P, i, P, i, P, P, P, i, i64, i64, i64, P]
    L.fp8_gemm_kmajor.argtypes = [P, i, i32, P, i, i32, P, P, P, i, i64, i64, i64, P]
    L.fp8_linear_copies.argtypes = [i64, i64, i64, P, P, P]
    L.fp8_gemm_kmajor_unscale.argtypes = [P, i, i32, P, i, i32, P, P, P, P, P, i64, i64, i64, P]
    L.fp8_scaled_linear_fwd.argtypes = [P, P, i64, i64, i64, ctypes.POINTER(_Saved), P, i, P]
    L.fp8_scaled_linear_bwd.argtypes = [P, ctypes.POINTER(_Saved), i64, i64, i64,
                                        ctypes.POINTER(_BwdWs), P, P, i, P]
    L.fp8_scaled_linear_fwd_delayed.argtypes = [P, P, i64, i64, i64, ctypes.POINTER(_Saved), P, P,
                                                i32, P, i, P]
    L.fp8_scaled_linear_bwd_delayed.argtypes = [P, ctypes.POINTER(_Saved), i64, i64, i64,
                                                ctypes.POINTER(_BwdWs), P, i32, P, P, i, P]
    L.amp_unscale_check.argtypes = [ctypes.POINTER(P), ctypes.POINTER(i64), i32, P, P, P]
    L.amp_update_scale.argtypes = [P, P, P, f32, f32, i32, P]
    L.amp_norm_workspace_len.argtypes = [ctypes.POINTER(i64), i32]
    L.amp_norm_workspace_len.restype = i64
    L.amp_unscale_check_norm_noalloc.argtypes = [ctypes.POINTER(P), ctypes.POINTER(i64), i32, P,
                                                 P, P, P]
    L.amp_unscale_check_norm.argtypes = [ctypes.POINTER(P), ctypes.POINTER(i64), i32, P, P, P, i64,
                                         P, P]
    L.fp8_quantize_rowwise.argtypes = [P, i64, i64, i, P, P, P, P, P, P, P]
    L.fp8_gemm_rowwise.argtypes = [P, i, P, i, P, P, P, i, i64, i64, i64, P]
    L.fp8_scaled_linear_fwd_rowwise.argtypes = [P, P, i64, i64, i64, ctypes.POINTER(_SavedRW), P,
                                                i, P]
    L.fp8_scaled_linear_bwd_rowwise.argtypes = [P, ctypes.POINTER(_SavedRW), i64, i64, i64,
                                                ctypes.POINTER(_BwdWsRW), P, P, i, P]
    L.fp8_gemm_unscale.argtypes = [P, i, P, i, P, P, P, P, P, i64, i64, i64, P]
    L.fp8_scaled_linear_bwd_unscale.argtypes = [P, ctypes.POINTER(_Saved), i64, i64, i64,
                                                ctypes.POINTER(_BwdWs), P, P, P, P, P]
    L.fp8_scaled_linear_bwd_delayed_unscale.argtypes = [P, ctypes.POINTER(_Saved), i64, i64, i64,
                                                        ctypes.POINTER(_BwdWs), P, i32, P, P, P,
                                                        P, P]
    L.fp8_scaled_linear_bwd_rowwise_unscale.argtypes = [P, ctypes.POINTER(_SavedRW), i64, i64, i64,
                                                        ctypes.POINTER(_BwdWsRW), P, P, P, P, P]
    for name in EXPORTS[3:]:
        getattr(L, name).restype = i
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        msg = lib().fp8sg_status_string(status).decode()
        raise Fp8sgError(f"{what}: status {status} ({msg})")


def _ptr(t):
    """Device address of a tensor (NULL for None); host tensors are refused."""
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError("tensor arguments must be device tensors")
    return ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    """hipStream_t of `stream`, or of torch's current stream on the current device."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None and _cur_device is not None:
        return ctypes.c_void_p(_raw_stream(_cur_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_OUT_DTYPE = {OUT_BF16: torch.bfloat16, OUT_F16: torch.float16, OUT_F32: torch.float32}


def _need(t, name, dtype, shape=None, numel=None, min_numel=None):
    """Refuses a tensor the library would read or write out of bounds.  The C
    ABI sees pointers and sizes only, so dtype, shape and contiguity are
    checked here, before any call (TypeError / ValueError); _ptr checks the
    device when the arguments are marshalled."""
    try:  # the common case in one expression; the checks below name what failed
        if ((dtype is None or t.dtype == dtype) and (shape is None or t.shape == shape)
                and (numel is None or t.numel() == numel)
                and (min_numel is None or t.numel() >= min_numel) and t.is_contiguous()):
            return
    except AttributeError:
        pass
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected at least {min_numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _need_rec(rec, name):
    if not isinstance(rec, ScaleRec):
        raise TypeError(f"{name}: expected a ScaleRec")
    _need(rec.buf, name, torch.uint8, min_numel=SCALE_REC_BYTES)


def _need_2d(t, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor")
    return t.shape


def _need_scaler(scale, found_inf):
    _need(scale, "scale", torch.float32, min_numel=1)
    _need(found_inf, "found_inf", torch.int32, min_numel=1)


# ----------------------------------------------------------------- scale records

class ScaleRec:
    """A device scale record (fp8sg_scale_rec, 4128 bytes).

    Fields (after the library has written them): amax, scale32, inv32 (fp32),
    scale, inv (fp64)."""

    def __init__(self, device="cuda", buf=None):
        self.buf = buf if buf is not None else torch.zeros(SCALE_REC_BYTES, dtype=torch.uint8,
                                                          device=device)

    @property
    def ptr(self):
        return self.buf.data_ptr()

    def inv_ptr(self):
        return self.buf.data_ptr() + 24

    def read(self) -> dict:
        h = self.buf[:32].cpu()
        f = h[:12].view(torch.float32)
        u = h[:16].view(torch.int32)
        d = h[16:32].view(torch.float64)
        return {"amax": float(f[0]), "scale32": float(f[1]), "inv32": float(f[2]),
                "amax_bits": int(u[0]) & 0xFFFFFFFF, "scale32_bits": int(u[1]) & 0xFFFFFFFF,
                "inv32_bits": int(u[2]) & 0xFFFFFFFF, "scale": float(d[0]), "inv": float(d[1]),
                "nparts": int(u[3])}


# ----------------------------------------------------------------- C-ABI calls

def fp8_amax(x: torch.Tensor, rec: ScaleRec, stream=None):
    """rec.amax = max |x| over a bf16 tensor (any shape, contiguous)."""
    _need(x, "x", torch.bfloat16)
    _need_rec(rec, "rec")
    _check(lib().fp8_amax(_ptr(x), x.numel(), _ptr(rec.buf), _stream(stream)),
           "fp8_amax")


def fp8_quantize(x: torch.Tensor, fmt: int, rec: ScaleRec, q: torch.Tensor,
                 qT: torch.Tensor = None, stream=None):
    """Scale from rec.amax, then codes q (= x's shape) and optionally qT (transposed)."""
    rows, cols = _quant_args(x, rec, q, qT)
    _check(lib().fp8_quantize(_ptr(x), rows, cols, fmt, _ptr(rec.buf), _ptr(q),
                              _ptr(qT), _stream(stream)), "fp8_quantize")


def fp8_amax_f16(x: torch.Tensor, rec: ScaleRec, stream=None):
    """rec.amax = max |x| over an fp16 tensor (any shape, contiguous)."""
    _need(x, "x", torch.float16)
    _need_rec(rec, "rec")
    _check(lib().fp8_amax_f16(_ptr(x), x.numel(), _ptr(rec.buf), _stream(stream)), "fp8_amax_f16")


def fp8_quantize_f16(x: torch.Tensor, fmt: int, rec: ScaleRec, q: torch.Tensor,
                     qT: torch.Tensor = None, stream=None):
    """fp8_quantize for an fp16 tensor: scale from rec.amax (fp8_amax_f16), codes q
    (and the transposed codes qT)."""
    _need(x, "x", torch.float16)
    _need_rec(rec, "rec")
    _need(q, "q", torch.uint8, numel=x.numel())
    if qT is not None:
        _need(qT, "qT", torch.uint8, numel=x.numel())
    rows, cols = (x.shape[0], x.numel() // max(x.shape[0], 1)) if x.dim() >= 2 else (1, x.numel())
    _check(lib().fp8_quantize_f16(_ptr(x), rows, cols, fmt, _ptr(rec.buf), _ptr(q), _ptr(qT),
                                  _stream(stream)), "fp8_quantize_f16")


def fp8_quantize_from_amax(x: torch.Tensor, fmt: int, amax: torch.Tensor, rec: ScaleRec,
                           q: torch.Tensor, qT: torch.Tensor = None, stream=None):
    """Scale from the caller's amax (a one-element device float32 tensor), then
    codes q (= x's shape) and optionally qT; rec receives amax and the scales."""
    rows, cols = _quant_args(x, rec, q, qT)
    _need(amax, "amax", torch.float32, numel=1)
    _check(lib().fp8_quantize_from_amax(_ptr(x), rows, cols, fmt, _ptr(amax), _ptr(rec.buf),
                                        _ptr(q), _ptr(qT), _stream(stream)),
           "fp8_quantize_from_amax")


def _quant_args(x, rec, q, qT):
    _need(x, "x", torch.bfloat16)
    _need_rec(rec, "rec")
    _need(q, "q", torch.uint8, numel=x.numel())
    if qT is not None:
        _need(qT, "qT", torch.uint8, numel=x.numel())
    return (x.shape[0], x.numel() // max(x.shape[0], 1)) if x.dim() >= 2 else (1, x.numel())


def _hist(h: torch.Tensor, name="hist"):
    _need(h, name, torch.float32)
    if not 1 <= h.numel() <= MAX_HISTORY:
        raise ValueError(f"{name}: history length {h.numel()} outside 1..{MAX_HISTORY}")
    return h.numel()


def fp8_quantize_delayed(x: torch.Tensor, fmt: int, rec: ScaleRec, hist: torch.Tensor,
                         q: torch.Tensor, qT: torch.Tensor = None, stream=None):
    """Delayed scaling: scale from the largest entry of the amax history hist
    (device float32, most recent first), codes q (and qT), then rec.amax =
    max |x| pushed to the front of hist."""
    rows, cols = _quant_args(x, rec, q, qT)
    h = _hist(hist)
    _check(lib().fp8_quantize_delayed(_ptr(x), rows, cols, fmt, _ptr(hist), h,
                                      _ptr(rec.buf), _ptr(q), _ptr(qT),
                                      _stream(stream)), "fp8_quantize_delayed")


def _gemm_args(A, B, C, c_dtype):
    M, K = _need_2d(A, "A")
    N, K2 = _need_2d(B, "B")
    _need(A, "A", torch.uint8)
    _need(B, "B", torch.uint8, shape=(N, K))
    _need(C, "C", c_dtype, shape=(M, N))
    return M, N, K


def fp8_gemm(A: torch.Tensor, fa: int, B: torch.Tensor, fb: int, inv_a_ptr: int, inv_b_ptr: int,
             C: torch.Tensor, out: int, stream=None):
    """C[M,N] = A[M,K] . B[N,K]^T * fl32(inv_a * inv_b); inv_*_ptr are device double addresses."""
    M, N, K = _gemm_args(A, B, C, _OUT_DTYPE.get(out))
    _check(lib().fp8_gemm(_ptr(A), fa, _ptr(B), fb, ctypes.c_void_p(inv_a_ptr),
                          ctypes.c_void_p(inv_b_ptr), _ptr(C), out, M, N, K, _stream(stream)),
           "fp8_gemm")


def fp8_gemm_unscale(A: torch.Tensor, fa: int, B: torch.Tensor, fb: int, inv_a_ptr: int,
                     inv_b_ptr: int, scale: torch.Tensor, found_inf: torch.Tensor, C: torch.Tensor,
                     stream=None):
    """fp8_gemm into fp16 C with the GradScaler unscale and check in the epilogue."""
    M, N, K = _gemm_args(A, B, C, torch.float16)
    _need_scaler(scale, found_inf)
    _check(lib().fp8_gemm_unscale(_ptr(A), fa, _ptr(B), fb, ctypes.c_void_p(inv_a_ptr),
                                  ctypes.c_void_p(inv_b_ptr), _ptr(scale), _ptr(found_inf), _ptr(C),
                                  M, N, K, _stream(stream)), "fp8_gemm_unscale")


def _kmajor_args(A, a_kmajor, B, b_kmajor, C, c_dtype):
    """Shapes of a GEMM whose operands may be stored contraction-major."""
    a0, a1 = _need_2d(A, "A")
    b0, b1 = _need_2d(B, "B")
    M, K = (a1, a0) if a_kmajor else (a0, a1)
    N = b1 if b_kmajor else b0
    _need(A, "A", torch.uint8)
    _need(B, "B", torch.uint8, shape=(K, N) if b_kmajor else (N, K))
    _need(C, "C", c_dtype, shape=(M, N))
    return M, N, K


def fp8_gemm_kmajor(A: torch.Tensor, fa: int, a_kmajor: bool, B: torch.Tensor, fb: int,
                    b_kmajor: bool, inv_a_ptr: int, inv_b_ptr: int, C: torch.Tensor, out: int,
                    stream=None):
    """fp8_gemm with A given as A^T [K, M] (a_kmajor) and/or B as B^T [K, N]
    (b_kmajor), read in that layout: the backward GEMMs on row-major codes."""
    M, N, K = _kmajor_args(A, a_kmajor, B, b_kmajor, C, _OUT_DTYPE.get(out))
    _check(lib().fp8_gemm_kmajor(_ptr(A), fa, int(bool(a_kmajor)), _ptr(B), fb, int(bool(b_kmajor)),
                                 ctypes.c_void_p(inv_a_ptr), ctypes.c_void_p(inv_b_ptr), _ptr(C), out,
                                 M, N, K, _stream(stream)), "fp8_gemm_kmajor")


def fp8_gemm_kmajor_unscale(A: torch.Tensor, fa: int, a_kmajor: bool, B: torch.Tensor, fb: int,
                            b_kmajor: bool, inv_a_ptr: int, inv_b_ptr: int, scale: torch.Tensor,
                            found_inf: torch.Tensor, C: torch.Tensor, stream=None):
    """fp8_gemm_unscale with contraction-major operands (as fp8_gemm_kmajor)."""
    M, N, K = _kmajor_args(A, a_kmajor, B, b_kmajor, C, torch.float16)
    _need_scaler(scale, found_inf)
    _check(lib().fp8_gemm_kmajor_unscale(_ptr(A), fa, int(bool(a_kmajor)), _ptr(B), fb,
                                         int(bool(b_kmajor)), ctypes.c_void_p(inv_a_ptr),
                                         ctypes.c_void_p(inv_b_ptr), _ptr(scale), _ptr(found_inf),
                                         _ptr(C), M, N, K, _stream(stream)), "fp8_gemm_kmajor_unscale")


_copies_cache = {}


def fp8_linear_copies(M: int, N: int, K: int):
    """(x_T, w_T, gy_T): which transposed copies make the backward of an
    M x N x K linear layer fastest on the current device (the results are the
    same bits with any choice).  Cached per device and size."""
    key = (torch.cuda.current_device() if torch.cuda.is_available() else -1, M, N, K)
    got = _copies_cache.get(key)
    if got is None:
        v = [ctypes.c_int32(0) for _ in range(3)]
        _check(lib().fp8_linear_copies(M, N, K, *[ctypes.addressof(a) for a in v]),
               "fp8_linear_copies")
        got = _copies_cache[key] = tuple(bool(a.value) for a in v)
    return got


class LinearSaved:
    """Device buffers the forward pass fills for the backward pass.  With
    transposed=False no transposed copies are kept (x_qT and w_qT are None):
    the backward GEMMs read x_q and w_q contraction-major.  x_transposed /
    w_transposed choose for one operand alone (default: `transposed`)."""

    def __init__(self, M, N, K, device="cuda", tensors=None, transposed=True, x_transposed=None,
                 w_transposed=None):
        if tensors is not None:  # (x_q, x_qT, w_q, w_qT, recs) kept from an earlier forward
            self.x_q, self.x_qT, self.w_q, self.w_qT, self.recs = tensors
        else:
            xt = transposed if x_transposed is None else x_transposed
            wt = transposed if w_transposed is None else w_transposed
            u8 = dict(dtype=torch.uint8, device=device)
            self.x_q = torch.empty((M, K), **u8)
            self.x_qT = torch.empty((K, M), **u8) if xt else None
            self.w_q = torch.empty((N, K), **u8)
            self.w_qT = torch.empty((K, N), **u8) if wt else None
            self.recs = torch.zeros((2, SCALE_REC_BYTES), **u8)
        self.x_sc = ScaleRec(buf=self.recs[0])
        self.w_sc = ScaleRec(buf=self.recs[1])

    def tensors(self):
        return (self.x_q, self.x_qT, self.w_q, self.w_qT, self.recs)

    def check(self, M, N, K):
        """The buffers must fit a layer of these sizes (checked once per set of
        buffer objects and sizes)."""
        key = (M, N, K, id(self.x_q), id(self.x_qT), id(self.w_q), id(self.w_qT), id(self.x_sc),
               id(self.w_sc), id(self.x_sc.buf), id(self.w_sc.buf))
        if self.__dict__.get("_ok") == key:
            return
        for t, name, shape in ((self.x_q, "saved.x_q", (M, K)), (self.x_qT, "saved.x_qT", (K, M)),
                               (self.w_q, "saved.w_q", (N, K)), (self.w_qT, "saved.w_qT", (K, N))):
            if t is not None or name in ("saved.x_q", "saved.w_q"):
                _need(t, name, torch.uint8, shape=shape)
        _need_rec(self.x_sc, "saved.x_sc")
        _need_rec(self.w_sc, "saved.w_sc")
        self._ok = key

    def struct(self):
        """The C struct, rebuilt only when check() has seen other buffers."""
        ok = self.__dict__.get("_ok")
        if ok is None or self.__dict__.get("_st_key") != ok:
            self._st, self._st_key = self._build(), ok
        return self._st

    def _build(self):
        return _Saved(*[_ptr(t).value for t in (self.x_q, self.x_qT, self.w_q, self.w_qT,
                                                  self.x_sc.buf, self.w_sc.buf)])


class LinearBwdWs:
    """The backward's gradient codes; with transposed=False no transposed copy
    (the weight-gradient GEMM then reads gy_q contraction-major).  gy_sc: the
    scale record to use (default: a new zeroed one)."""

    def __init__(self, M, N, device="cuda", transposed=True, gy_sc=None):
        u8 = dict(dtype=torch.uint8, device=device)
        self.gy_q = torch.empty((M, N), **u8)
        self.gy_qT = torch.empty((N, M), **u8) if transposed else None
        self.gy_sc = gy_sc if gy_sc is not None else ScaleRec(device=device)

    def check(self, M, N):
        key = (M, N, id(self.gy_q), id(self.gy_qT), id(self.gy_sc), id(self.gy_sc.buf))
        if self.__dict__.get("_ok") == key:
            return
        _need(self.gy_q, "ws.gy_q", torch.uint8, shape=(M, N))
        if self.gy_qT is not None:
            _need(self.gy_qT, "ws.gy_qT", torch.uint8, shape=(N, M))
        _need_rec(self.gy_sc, "ws.gy_sc")
        self._ok = key

    def struct(self):
        ok = self.__dict__.get("_ok")
        if ok is None or self.__dict__.get("_st_key") != ok:
            self._st, self._st_key = self._build(), ok
        return self._st

    def _build(self):
        return _BwdWs(*[_ptr(t).value for t in (self.gy_q, self.gy_qT, self.gy_sc.buf)])


def _fwd_args(x, w, y, out):
    M, K = _need_2d(x, "x")
    N, _ = _need_2d(w, "w")
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16, shape=(N, K))
    _need(y, "y", _OUT_DTYPE.get(out), shape=(M, N))
    return M, N, K


def _bwd_args(gy, saved, gx, gw, out):
    M, N = _need_2d(gy, "gy")
    _need(gy, "gy", torch.bfloat16)
    K = _need_2d(saved.x_q, "saved.x_q")[1]
    dt = _OUT_DTYPE.get(out)
    _need(gx, "gx", dt, shape=(M, K))
    _need(gw, "gw", dt, shape=(N, K))
    return M, N, K


def fp8_scaled_linear_fwd(x, w, saved: LinearSaved, y, out: int = OUT_BF16, stream=None):
    M, N, K = _fwd_args(x, w, y, out)
    saved.check(M, N, K)
    s = saved.struct()
    _check(lib().fp8_scaled_linear_fwd(_ptr(x), _ptr(w), M, N, K, ctypes.byref(s), _ptr(y), out,
                                       _stream(stream)), "fp8_scaled_linear_fwd")


def fp8_scaled_linear_bwd(gy, saved: LinearSaved, ws: LinearBwdWs, gx, gw, out: int = OUT_BF16,
                          stream=None):
    M, N, K = _bwd_args(gy, saved, gx, gw, out)
    saved.check(M, N, K)
    ws.check(M, N)
    s = saved.struct()
    b = ws.struct()
    _check(lib().fp8_scaled_linear_bwd(_ptr(gy), ctypes.byref(s), M, N, K, ctypes.byref(b),
                                       _ptr(gx), _ptr(gw), out, _stream(stream)),
           "fp8_scaled_linear_bwd")


def fp8_scaled_linear_bwd_unscale(gy, saved: LinearSaved, ws: LinearBwdWs, scale, found_inf,
                                  gx, gw, stream=None):
    """fp8_scaled_linear_bwd into fp16 gx, gw with the GradScaler unscale and
    non-finite check fused into the GEMM epilogues."""
    M, N, K = _bwd_args(gy, saved, gx, gw, OUT_F16)
    _need_scaler(scale, found_inf)
    saved.check(M, N, K)
    ws.check(M, N)
    s = saved.struct()
    b = ws.struct()
    _check(lib().fp8_scaled_linear_bwd_unscale(_ptr(gy), ctypes.byref(s), M, N, K, ctypes.byref(b),
                                               _ptr(scale), _ptr(found_inf), _ptr(gx), _ptr(gw),
                                               _stream(stream)), "fp8_scaled_linear_bwd_unscale")


def fp8_scaled_linear_fwd_delayed(x, w, saved: LinearSaved, hist_x, hist_w, y,
                                  out: int = OUT_BF16, stream=None):
    M, N, K = _fwd_args(x, w, y, out)
    h = _hist(hist_x, "hist_x")
    if _hist(hist_w, "hist_w") != h:
        raise ValueError("hist_x and hist_w must have the same length")
    saved.check(M, N, K)
    s = saved.struct()
    _check(lib().fp8_scaled_linear_fwd_delayed(_ptr(x), _ptr(w), M, N, K, ctypes.byref(s),
                                               _ptr(hist_x), _ptr(hist_w), h, _ptr(y), out,
                                               _stream(stream)), "fp8_scaled_linear_fwd_delayed")


def fp8_scaled_linear_bwd_delayed(gy, saved: LinearSaved, ws: LinearBwdWs, hist_gy, gx, gw,
                                  out: int = OUT_BF16, stream=None):
    M, N, K = _bwd_args(gy, saved, gx, gw, out)
    saved.check(M, N, K)
    ws.check(M, N)
    s = saved.struct()
    b = ws.struct()
    _check(lib().fp8_scaled_linear_bwd_delayed(_ptr(gy), ctypes.byref(s), M, N, K, ctypes.byref(b),
                                               _ptr(hist_gy), _hist(hist_gy, "hist_gy"), _ptr(gx),
                                               _ptr(gw),
                                               out, _stream(stream)),
           "fp8_scaled_linear_bwd_delayed")


def fp8_scaled_linear_bwd_delayed_unscale(gy, saved: LinearSaved, ws: LinearBwdWs, hist_gy,
                                          scale, found_inf, gx, gw, stream=None):
    """fp8_scaled_linear_bwd_delayed into fp16 gx, gw with the GradScaler
    unscale and non-finite check fused into the GEMM epilogues."""
    M, N, K = _bwd_args(gy, saved, gx, gw, OUT_F16)
    _need_scaler(scale, found_inf)
    h = _hist(hist_gy, "hist_gy")
    saved.check(M, N, K)
    ws.check(M, N)
    s = saved.struct()
    b = ws.struct()
    _check(lib().fp8_scaled_linear_bwd_delayed_unscale(
        _ptr(gy), ctypes.byref(s), M, N, K, ctypes.byref(b), _ptr(hist_gy), h, _ptr(scale),
        _ptr(found_inf), _ptr(gx), _ptr(gw), _stream(stream)), "fp8_scaled_linear_bwd_delayed_unscale")


# ----------------------------------------------------------------- row-wise

class RowScalesDev:
    """A row-wise scale-vector pair: amax float32[n], inv float64[n]."""

    def __init__(self, n, device="cuda", amax=None, inv=None):
        self.amax = amax if amax is not None else torch.empty(n, dtype=torch.float32, device=device)
        self.inv = inv if inv is not None else torch.empty(n, dtype=torch.float64, device=device)


def _need_vec(sc, name, n):
    if not isinstance(sc, RowScalesDev):
        raise TypeError(f"{name}: expected a RowScalesDev")
    _need(sc.amax, name + ".amax", torch.float32, numel=n)
    _need(sc.inv, name + ".inv", torch.float64, numel=n)


def fp8_quantize_rowwise(x: torch.Tensor, fmt: int, rows_sc: RowScalesDev, q: torch.Tensor,
                         cols_sc: RowScalesDev = None, qT: torch.Tensor = None, stream=None):
    """Row-wise cast of a [rows, cols] bf16 matrix: q with one scale per row
    (rows_sc), and with qT the transposed copy with one scale per column
    (cols_sc)."""
    rows, cols = _need_2d(x, "x")
    _need(x, "x", torch.bfloat16)
    _need(q, "q", torch.uint8, shape=(rows, cols))
    _need_vec(rows_sc, "rows_sc", rows)
    if cols_sc is not None or qT is not None:
        _need_vec(cols_sc, "cols_sc", cols)
        _need(qT, "qT", torch.uint8, shape=(cols, rows))
    ca = cols_sc.amax if cols_sc is not None else None
    ci = cols_sc.inv if cols_sc is not None else None
    _check(lib().fp8_quantize_rowwise(_ptr(x), rows, cols, fmt, _ptr(rows_sc.amax),
                                      _ptr(rows_sc.inv), _ptr(q), _ptr(ca), _ptr(ci), _ptr(qT),
                                      _stream(stream)), "fp8_quantize_rowwise")


def fp8_gemm_rowwise(A: torch.Tensor, fa: int, B: torch.Tensor, fb: int, inv_a: torch.Tensor,
                     inv_b: torch.Tensor, C: torch.Tensor, out: int, stream=None):
    """C[M,N] = A[M,K] . B[N,K]^T * fl32(inv_a[m] * inv_b[n]) (float64 vectors)."""
    M, N, K = _gemm_args(A, B, C, _OUT_DTYPE.get(out))
    _need(inv_a, "inv_a", torch.float64, numel=M)
    _need(inv_b, "inv_b", torch.float64, numel=N)
    _check(lib().fp8_gemm_rowwise(_ptr(A), fa, _ptr(B), fb, _ptr(inv_a), _ptr(inv_b), _ptr(C),
                                  out, M, N, K, _stream(stream)), "fp8_gemm_rowwise")


class LinearSavedRW:
    """Device buffers the row-wise forward fills for the backward pass: codes
    of x and W by rows and (transposed) by columns, with their scale vectors."""

    NAMES = ("x_q", "x_qT", "w_q", "w_qT", "x_row_amax", "x_row_inv", "x_col_amax", "x_col_inv",
             "w_row_amax", "w_row_inv", "w_col_amax", "w_col_inv")

    def __init__(self, M, N, K, device="cuda", tensors=None):
        if tensors is None:
            u8 = dict(dtype=torch.uint8, device=device)
            f32 = dict(dtype=torch.float32, device=device)
            f64 = dict(dtype=torch.float64, device=device)
            tensors = (torch.empty((M, K), **u8), torch.empty((K, M), **u8),
                       torch.empty((N, K), **u8), torch.empty((K, N), **u8),
                       torch.empty(M, **f32), torch.empty(M, **f64),
                       torch.empty(K, **f32), torch.empty(K, **f64),
                       torch.empty(N, **f32), torch.empty(N, **f64),
                       torch.empty(K, **f32), torch.empty(K, **f64))
        for n, t in zip(self.NAMES, tensors):
            setattr(self, n, t)

    def tensors(self):
        return tuple(getattr(self, n) for n in self.NAMES)

    def check(self, M, N, K):
        key = (M, N, K) + tuple(id(getattr(self, n)) for n in self.NAMES)
        if self.__dict__.get("_ok") == key:
            return
        shapes = ((M, K), (K, M), (N, K), (K, N), (M,), (M,), (K,), (K,), (N,), (N,), (K,), (K,))
        for n, shape in zip(self.NAMES, shapes):
            dt = torch.uint8 if len(shape) == 2 else (
                torch.float32 if n.endswith("amax") else torch.float64)
            _need(getattr(self, n), "saved." + n, dt, shape=shape)
        self._ok = key

    def struct(self):
        ok = self.__dict__.get("_ok")
        if ok is None or self.__dict__.get("_st_key") != ok:
            self._st, self._st_key = self._build(), ok
        return self._st

    def _build(self):
        return _SavedRW(*[_ptr(getattr(self, n)).value for n in self.NAMES])


class LinearBwdWsRW:
    NAMES = ("gy_q", "gy_qT", "gy_row_amax", "gy_row_inv", "gy_col_amax", "gy_col_inv")

    def __init__(self, M, N, device="cuda"):
        u8 = dict(dtype=torch.uint8, device=device)
        self.gy_q = torch.empty((M, N), **u8)
        self.gy_qT = torch.empty((N, M), **u8)
        self.gy_row_amax = torch.empty(M, dtype=torch.float32, device=device)
        self.gy_row_inv = torch.empty(M, dtype=torch.float64, device=device)
        self.gy_col_amax = torch.empty(N, dtype=torch.float32, device=device)
        self.gy_col_inv = torch.empty(N, dtype=torch.float64, device=device)

    def check(self, M, N):
        key = (M, N) + tuple(id(getattr(self, n)) for n in self.NAMES)
        if self.__dict__.get("_ok") == key:
            return
        shapes = ((M, N), (N, M), (M,), (M,), (N,), (N,))
        dts = (torch.uint8, torch.uint8, torch.float32, torch.float64, torch.float32, torch.float64)
        for n, shape, dt in zip(self.NAMES, shapes, dts):
            _need(getattr(self, n), "ws." + n, dt, shape=shape)
        self._ok = key

    def struct(self):
        ok = self.__dict__.get("_ok")
        if ok is None or self.__dict__.get("_st_key") != ok:
            self._st, self._st_key = self._build(), ok
        return self._st

    def _build(self):
        return _BwdWsRW(*[_ptr(getattr(self, n)).value for n in self.NAMES])


def fp8_scaled_linear_fwd_rowwise(x, w, saved: LinearSavedRW, y, out: int = OUT_BF16,
                                  stream=None):
    M, N, K = _fwd_args(x, w, y, out)
    saved.check(M, N, K)
    s = saved.struct()
    _check(lib().fp8_scaled_linear_fwd_rowwise(_ptr(x), _ptr(w), M, N, K, ctypes.byref(s),
                                               _ptr(y), out, _stream(stream)),
           "fp8_scaled_linear_fwd_rowwise")


def fp8_scaled_linear_bwd_rowwise(gy, saved: LinearSavedRW, ws: LinearBwdWsRW, gx, gw,
                                  out: int = OUT_BF16, stream=None):
    M, N, K = _bwd_args(gy, saved, gx, gw, out)
    saved.check(M, N, K)
    ws.check(M, N)
    s = saved.struct()
    b = ws.struct()
    _check(lib().fp8_scaled_linear_bwd_rowwise(_ptr(gy), ctypes.byref(s), M, N, K,
                                               ctypes.byref(b), _ptr(gx), _ptr(gw), out,
                                               _stream(stream)), "fp8_scaled_linear_bwd_rowwise")


def fp8_scaled_linear_bwd_rowwise_unscale(gy, saved: LinearSavedRW, ws: LinearBwdWsRW, scale,
                                          found_inf, gx, gw, stream=None):
    """fp8_scaled_linear_bwd_rowwise into fp16 gx, gw with the GradScaler
    unscale and non-finite check fused into the GEMM epilogues."""
    M, N, K = _bwd_args(gy, saved, gx, gw, OUT_F16)
    _need_scaler(scale, found_inf)
    saved.check(M, N, K)
    ws.check(M, N)
    s = saved.struct()
    b = ws.struct()
    _check(lib().fp8_scaled_linear_bwd_rowwise_unscale(
        _ptr(gy), ctypes.byref(s), M, N, K, ctypes.byref(b), _ptr(scale), _ptr(found_inf),
        _ptr(gx), _ptr(gw), _stream(stream)), "fp8_scaled_linear_bwd_rowwise_unscale")


def _grad_list(grads):
    grads = list(grads)
    for i, g in enumerate(grads):
        _need(g, f"grads[{i}]", torch.float16)
    n = len(grads)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(g).value for g in grads])
    numel = (ctypes.c_int64 * max(n, 1))(*[g.numel() for g in grads])
    return ptrs, numel, n


def amp_unscale_check(grads, scale: torch.Tensor, found_inf: torch.Tensor, stream=None):
    """In-place unscale of a list of fp16 gradients and OR of the non-finite flag."""
    ptrs, numel, n = _grad_list(grads)
    _need_scaler(scale, found_inf)
    _check(lib().amp_unscale_check(ptrs, numel, n, _ptr(scale), _ptr(found_inf),
                                   _stream(stream)), "amp_unscale_check")


def amp_norm_workspace_len(numels) -> int:
    """fp32 slots amp_unscale_check_norm needs for tensors of these sizes."""
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in numels])
    r = lib().amp_norm_workspace_len(arr, n)
    if r < 0:
        raise Fp8sgError(f"amp_norm_workspace_len: invalid sizes {list(numels)[:4]}...")
    return int(r)


def amp_unscale_check_norm(grads, scale: torch.Tensor, found_inf: torch.Tensor,
                           workspace: torch.Tensor, sumsq_norm: torch.Tensor, stream=None):
    """amp_unscale_check plus (sum of squares, 2-norm) of the unscaled gradients
    into sumsq_norm (device float32[2]); workspace: device float32 scratch of at
    least amp_norm_workspace_len([g.numel() for g in grads]) elements."""
    ptrs, numel, n = _grad_list(grads)
    _need_scaler(scale, found_inf)
    _need(workspace, "workspace", torch.float32)
    _need(sumsq_norm, "sumsq_norm", torch.float32, min_numel=2)
    _check(lib().amp_unscale_check_norm(ptrs, numel, n, _ptr(scale), _ptr(found_inf),
                                        _ptr(workspace), workspace.numel(), _ptr(sumsq_norm),
                                        _stream(stream)), "amp_unscale_check_norm")


NOALLOC_NORM_SLOTS = 1 << 20  # FP8SG_NOALLOC_NORM_SLOTS


def amp_unscale_check_norm_noalloc(grads, scale: torch.Tensor, found_inf: torch.Tensor,
                                   sumsq_norm: torch.Tensor, stream=None):
    """amp_unscale_check_norm without a workspace: the library's fixed scratch
    array (one per GPU) holds the partial sums; nothing is allocated.  Calls
    that overlap in time on one GPU race."""
    ptrs, numel, n = _grad_list(grads)
    _need_scaler(scale, found_inf)
    _need(sumsq_norm, "sumsq_norm", torch.float32, min_numel=2)
    _check(lib().amp_unscale_check_norm_noalloc(ptrs, numel, n, _ptr(scale), _ptr(found_inf),
                                                _ptr(sumsq_norm), _stream(stream)),
           "amp_unscale_check_norm_noalloc")


def amp_update_scale(scale: torch.Tensor, growth_tracker: torch.Tensor, found_inf: torch.Tensor,
                     growth_factor=2.0, backoff_factor=0.5, growth_interval=2000, stream=None):
    _need_scaler(scale, found_inf)
    _need(growth_tracker, "growth_tracker", torch.int32, min_numel=1)
    _check(lib().amp_update_scale(_ptr(scale), _ptr(growth_tracker), _ptr(found_inf),
                                  growth_factor, backoff_factor, growth_interval, _stream(stream)),
           "amp_update_scale")
