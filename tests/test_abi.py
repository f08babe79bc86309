"""The C-ABI library loads on a machine without a GPU, exports every entry point
include/fp8sg.h declares, and rejects bad arguments before enqueuing anything.

Only validation paths run here (they return before any HIP call); compute calls
need a GPU and live in the gpu-marked tests.
"""
import ctypes
import os
import re

import pytest

import fp8_scaled_gemm_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8sg.h")

OK, ENULL, ESHAPE, EALIGN, EFORMAT = 0, 1, 2, 3, 4
A16 = 0x10000  # fake, never dereferenced: validation fails before any use
A16B = 0x20000
MIS = 0x10008  # not 16-byte aligned


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FP8SG_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    assert syms == sorted(F.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = F.lib()
    for s in declared_symbols():
        assert hasattr(L, s), s
    assert F.lib().fp8sg_version() >= 100
    for code in range(6):
        assert F.lib().fp8sg_status_string(code)


def test_scale_record_layout_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct fp8sg_scale_rec \{(.*?)\} fp8sg_scale_rec;", text, re.S).group(1)
    parts = int(re.search(r"#define FP8SG_AMAX_PARTS (\d+)", text).group(1))
    assert parts == F.AMAX_PARTS
    fields = re.findall(r"^\s*(float|double|uint32_t)\s+(\w+)(\[\w+\])?;", body, re.M)
    ctype = {"float": ctypes.c_float, "double": ctypes.c_double, "uint32_t": ctypes.c_uint32}

    class Rec(ctypes.Structure):
        _fields_ = [(n, ctype[t] * parts) if a else (n, ctype[t]) for t, n, a in fields]
    assert ctypes.sizeof(Rec) == F.SCALE_REC_BYTES == 32 + 4 * parts
    assert Rec.inv.offset == 24  # the binding hands &rec->inv to fp8_gemm


def P(v):
    return ctypes.c_void_p(v)


def test_f16_cast_validation():
    L = F.lib()
    assert L.fp8_amax_f16(P(A16), 16, P(0), P(0)) == ENULL
    assert L.fp8_amax_f16(P(0), 16, P(A16), P(0)) == ENULL
    assert L.fp8_amax_f16(P(A16), -1, P(A16), P(0)) == ESHAPE
    assert L.fp8_amax_f16(P(MIS), 16, P(A16), P(0)) == EALIGN
    q = L.fp8_quantize_f16
    assert q(P(A16), 4, 4, 7, P(A16), P(A16), P(0), P(0)) == EFORMAT
    assert q(P(A16), -1, 4, 0, P(A16), P(A16), P(0), P(0)) == ESHAPE
    assert q(P(A16), 4, 4, 0, P(0), P(A16), P(0), P(0)) == ENULL
    assert q(P(A16), 4, 4, 0, P(A16), P(A16), P(MIS), P(0)) == EALIGN


def test_noalloc_norm_validation():
    """amp_unscale_check_norm_noalloc refuses, before any launch, a list that
    needs more than the scratch's FP8SG_NOALLOC_NORM_SLOTS slots, and bad
    arguments (fake pointers: validation returns before any use)."""
    L = F.lib()
    f = L.amp_unscale_check_norm_noalloc
    n = 11 * 10 ** 9 // 8  # 8 tensors of 1.375e9 elements: about 1.34e6 blocks
    ptrs = (ctypes.c_void_p * 8)(*([A16] * 8))
    big = (ctypes.c_int64 * 8)(*([n] * 8))
    assert f(ptrs, big, 8, P(A16), P(A16), P(A16), P(0)) == ESHAPE
    assert F.amp_norm_workspace_len([n] * 8) > F.NOALLOC_NORM_SLOTS
    one = (ctypes.c_int64 * 1)(1000)
    assert f(ptrs, one, 1, P(0), P(A16), P(A16), P(0)) == ENULL        # scale
    assert f(ptrs, one, 1, P(A16), P(A16), P(0), P(0)) == ENULL        # sumsq_norm
    assert f(ptrs, one, 1, P(A16 + 2), P(A16), P(A16), P(0)) == EALIGN  # scale 4-byte
    assert f(ptrs, one, 1, P(A16), P(A16), P(A16 + 2), P(0)) == EALIGN  # sumsq_norm 4-byte
    assert f(ptrs, one, -1, P(A16), P(A16), P(A16), P(0)) == ESHAPE
    odd = (ctypes.c_void_p * 1)(A16 + 1)
    assert f(odd, one, 1, P(A16), P(A16), P(A16), P(0)) == EALIGN      # fp16 needs 2-byte


def test_gemm_validation():
    L = F.lib()
    g = L.fp8_gemm
    args = [P(A16), 0, P(A16B), 0, P(A16), P(A16), P(A16B), 0, 16, 16, 16, P(0)]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return g(*a)

    assert call(a0=P(0)) == ENULL
    assert call(a4=P(0)) == ENULL
    assert call(a0=P(0), a4=P(0), a10=0) == ENULL  # Kc == 0 allows NULL A, never NULL scales
    assert call(a1=7) == EFORMAT
    assert call(a7=9) == EFORMAT
    assert call(a8=24) == ESHAPE
    assert call(a10=8) == ESHAPE
    assert call(a9=-16) == ESHAPE
    assert call(a0=P(MIS)) == EALIGN
    assert call(a6=P(MIS)) == EALIGN


def test_linear_and_quant_validation():
    L = F.lib()
    s = F._Saved(A16, A16, A16, A16, A16, A16)
    assert L.fp8_scaled_linear_fwd(P(A16), P(A16), 16, 16, 16, None, P(A16), 0, P(0)) == ENULL
    assert L.fp8_scaled_linear_fwd(P(A16), P(A16), 16, 15, 16, ctypes.byref(s), P(A16), 0, P(0)) == ESHAPE
    assert L.fp8_scaled_linear_fwd(P(A16), P(A16), 0, 16, 16, ctypes.byref(s), P(A16), 0, P(0)) == ESHAPE
    assert L.fp8_scaled_linear_fwd(P(MIS), P(A16), 16, 16, 16, ctypes.byref(s), P(A16), 0, P(0)) == EALIGN
    assert L.fp8_scaled_linear_fwd(P(A16), P(A16), 16, 16, 16, ctypes.byref(s), P(A16), 5, P(0)) == EFORMAT
    ws = F._BwdWs(A16, A16, 0)
    assert L.fp8_scaled_linear_bwd(P(A16), ctypes.byref(s), 16, 16, 16, ctypes.byref(ws), P(A16),
                                   P(A16), 0, P(0)) == ENULL
    assert L.fp8_quantize(P(A16), 4, 4, 3, P(A16), P(A16), P(0), P(0)) == EFORMAT
    assert L.fp8_quantize(P(A16), -1, 4, 0, P(A16), P(A16), P(0), P(0)) == ESHAPE
    assert L.fp8_quantize(P(A16), 4, 4, 0, P(A16), P(A16), P(MIS), P(0)) == EALIGN
    qa = L.fp8_quantize_from_amax
    assert qa(P(A16), 4, 4, 0, P(0), P(A16), P(A16), P(0), P(0)) == ENULL       # no amax
    assert qa(P(A16), 4, 4, 0, P(A16), P(0), P(A16), P(0), P(0)) == ENULL       # no record
    assert qa(P(0), 4, 4, 0, P(A16), P(A16), P(A16), P(0), P(0)) == ENULL       # no x
    assert qa(P(A16), 4, 4, 2, P(A16), P(A16), P(A16), P(0), P(0)) == EFORMAT
    assert qa(P(A16), -4, 4, 0, P(A16), P(A16), P(A16), P(0), P(0)) == ESHAPE
    assert qa(P(A16), 4, 4, 0, P(A16 + 2), P(A16), P(A16), P(0), P(0)) == EALIGN  # amax 4-byte
    assert qa(P(A16), 4, 4, 0, P(A16), P(A16 + 4), P(A16), P(0), P(0)) == EALIGN  # record 8-byte
    assert qa(P(A16), 4, 4, 0, P(A16), P(A16), P(A16), P(MIS), P(0)) == EALIGN   # qT 16-byte
    assert L.fp8_amax(P(0), 4, P(A16), P(0)) == ENULL
    assert L.fp8_amax(P(A16), -4, P(A16), P(0)) == ESHAPE
    assert L.fp8_amax(P(MIS), 4, P(A16), P(0)) == EALIGN


def test_amp_validation():
    L = F.lib()
    ptrs = (ctypes.c_void_p * 2)(A16, A16 + 1)  # fp16 needs 2-byte alignment only
    numel = (ctypes.c_int64 * 2)(8, 8)
    assert L.amp_unscale_check(ptrs, numel, 2, P(A16), P(A16), P(0)) == EALIGN
    numel[1] = -1
    assert L.amp_unscale_check(ptrs, numel, 2, P(A16), P(A16), P(0)) == ESHAPE
    assert L.amp_unscale_check(ptrs, numel, 2, P(0), P(A16), P(0)) == ENULL
    assert L.amp_unscale_check(ptrs, numel, 9000, P(A16), P(A16), P(0)) == ESHAPE
    assert L.amp_update_scale(P(A16), P(A16), P(A16), 2.0, 0.5, 0, P(0)) == ESHAPE
    assert L.amp_update_scale(P(0), P(A16), P(A16), 2.0, 0.5, 10, P(0)) == ENULL


def test_delayed_validation():
    L = F.lib()
    q = P(A16)
    # history length 0 and beyond the maximum; a NULL history; a misaligned one
    assert L.fp8_quantize_delayed(P(A16), 16, 16, 0, P(A16), 0, P(A16), q, q, P(0)) == ESHAPE
    assert L.fp8_quantize_delayed(P(A16), 16, 16, 0, P(A16), 1025, P(A16), q, q, P(0)) == ESHAPE
    assert L.fp8_quantize_delayed(P(A16), 16, 16, 0, P(0), 4, P(A16), q, q, P(0)) == ENULL
    assert L.fp8_quantize_delayed(P(A16), 16, 16, 0, P(A16 + 2), 4, P(A16), q, q, P(0)) == EALIGN
    assert L.fp8_quantize_delayed(P(A16), 16, 16, 7, P(A16), 4, P(A16), q, q, P(0)) == EFORMAT
    saved = F._Saved(A16, A16, A16, A16, A16, A16)
    ws = F._BwdWs(A16, A16, A16)
    fwd = lambda hx, hw, h: L.fp8_scaled_linear_fwd_delayed(P(A16), P(A16), 16, 16, 16,
                                                             ctypes.byref(saved), P(hx), P(hw), h,
                                                             P(A16), 0, P(0))
    assert fwd(0, A16, 4) == ENULL and fwd(A16, 0, 4) == ENULL
    assert fwd(A16, A16, 0) == ESHAPE and fwd(A16, A16 + 1, 4) == EALIGN
    bwd = lambda hg, h: L.fp8_scaled_linear_bwd_delayed(P(A16), ctypes.byref(saved), 16, 16, 16,
                                                        ctypes.byref(ws), P(hg), h, P(A16), P(A16),
                                                        0, P(0))
    assert bwd(0, 4) == ENULL and bwd(A16, 2000) == ESHAPE and bwd(A16 + 2, 4) == EALIGN


def test_norm_workspace_and_validation():
    L = F.lib()
    n = (ctypes.c_int64 * 3)(8192, 8193, 0)
    # ceil((numel + 7) / 8192) blocks per non-empty tensor (2 + 2 + 0), even, + 512
    assert L.amp_norm_workspace_len(n, 3) == 4 + 512
    n[2] = -1
    assert L.amp_norm_workspace_len(n, 3) == -1
    assert L.amp_norm_workspace_len(n, 9000) == -1
    ptrs = (ctypes.c_void_p * 2)(A16, A16 + 2)
    numel = (ctypes.c_int64 * 2)(8192, 8)
    need = 2 + 512  # the first tensor is aligned (one block), the second needs one more
    args = lambda ws_len, sn=A16, ws=A16: (ptrs, numel, 2, P(A16), P(A16), P(ws), ws_len, P(sn),
                                           P(0))
    assert L.amp_unscale_check_norm(*args(need - 1)) == ESHAPE
    assert L.amp_unscale_check_norm(*args(need, sn=0)) == ENULL
    assert L.amp_unscale_check_norm(*args(need, ws=0)) == ENULL
    assert L.amp_unscale_check_norm(*args(need, ws=A16 + 4)) == EALIGN
    assert L.amp_unscale_check_norm(*args(need, sn=A16 + 2)) == EALIGN
    ptrs[1] = A16 + 1
    assert L.amp_unscale_check_norm(*args(need)) == EALIGN


def test_rowwise_validation():
    L = F.lib()
    q = P(A16)
    quant = lambda rows=16, cols=32, fmt=0, ra=A16, ri=A16, ca=A16, ci=A16, qT=A16, x=A16: \
        L.fp8_quantize_rowwise(P(x), rows, cols, fmt, P(ra), P(ri), q, P(ca), P(ci), P(qT), P(0))
    assert quant(fmt=2) == EFORMAT
    assert quant(rows=8) == ESHAPE and quant(cols=-16) == ESHAPE
    assert quant(x=0) == ENULL and quant(ra=0) == ENULL and quant(ci=0) == ENULL
    assert quant(ra=A16 + 2) == EALIGN and quant(ri=A16 + 4) == EALIGN
    assert quant(ca=A16 + 1) == EALIGN and quant(qT=MIS) == EALIGN
    g = lambda ia=A16, ib=A16, M=16: L.fp8_gemm_rowwise(P(A16), 0, P(A16B), 1, P(ia), P(ib),
                                                        P(A16B), 0, M, 16, 32, P(0))
    assert g(ia=0) == ENULL and g(M=17) == ESHAPE and g(ib=A16 + 4) == EALIGN
    s = F._SavedRW(*([A16] * 12))
    ws = F._BwdWsRW(*([A16] * 6))
    fwd = lambda s, M=16: L.fp8_scaled_linear_fwd_rowwise(P(A16), P(A16), M, 16, 32,
                                                          ctypes.byref(s), P(A16), 0, P(0))
    bwd = lambda s, ws: L.fp8_scaled_linear_bwd_rowwise(P(A16), ctypes.byref(s), 16, 16, 32,
                                                        ctypes.byref(ws), P(A16), P(A16), 0, P(0))
    assert fwd(s, M=0) == ESHAPE
    for i, name in enumerate(F.LinearSavedRW.NAMES):
        bad = F._SavedRW(*([A16] * 12))
        setattr(bad, name, 0)
        assert fwd(bad) == ENULL, name
        setattr(bad, name, A16 + 2)
        assert fwd(bad) == EALIGN, name
        assert bwd(bad, ws) in (ENULL, EALIGN) and bwd(bad, ws) == EALIGN, name
    for name in F.LinearBwdWsRW.NAMES:
        bad = F._BwdWsRW(*([A16] * 6))
        setattr(bad, name, 0)
        assert bwd(s, bad) == ENULL, name


def test_fused_unscale_validation():
    L = F.lib()
    s = F._Saved(A16, A16, A16, A16, A16, A16)
    ws = F._BwdWs(A16, A16, A16)
    call = lambda scale=A16, found=A16, gx=A16, M=16: L.fp8_scaled_linear_bwd_unscale(
        P(A16), ctypes.byref(s), M, 16, 16, ctypes.byref(ws), P(scale), P(found), P(gx), P(A16),
        P(0))
    assert call(scale=0) == ENULL and call(found=0) == ENULL and call(gx=0) == ENULL
    assert call(scale=A16 + 2) == EALIGN and call(found=A16 + 1) == EALIGN
    assert call(gx=MIS) == EALIGN and call(M=8) == ESHAPE


def test_kmajor_validation():
    """The contraction-major GEMMs validate as fp8_gemm does; each of a linear
    layer's transposed copies (x_qT, w_qT, gy_qT) may be NULL on its own (a
    bad size after them shows the pointer checks passed, with no launch)."""
    L = F.lib()
    g = L.fp8_gemm_kmajor
    args = [P(A16), 0, 1, P(A16B), 0, 1, P(A16), P(A16), P(A16B), 0, 16, 32, 48, P(0)]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return g(*a)

    assert call(a0=P(0)) == ENULL and call(a3=P(0)) == ENULL and call(a6=P(0)) == ENULL
    assert call(a1=7) == EFORMAT and call(a9=9) == EFORMAT
    assert call(a10=24) == ESHAPE and call(a12=-16) == ESHAPE
    assert call(a0=P(MIS)) == EALIGN and call(a8=P(MIS)) == EALIGN
    u = lambda scale=A16, found=A16, C=A16B, M=16: L.fp8_gemm_kmajor_unscale(
        P(A16), 1, 1, P(A16B), 0, 1, P(A16), P(A16), P(scale), P(found), P(C), M, 16, 32, P(0))
    assert u(scale=0) == ENULL and u(found=0) == ENULL and u(C=0) == ENULL
    assert u(M=24) == ESHAPE and u(scale=A16 + 1) == EALIGN
    fwd = lambda s, M: L.fp8_scaled_linear_fwd(P(A16), P(A16), M, 16, 16, ctypes.byref(s),
                                               P(A16), 0, P(0))
    bwd = lambda s, ws, M: L.fp8_scaled_linear_bwd(P(A16), ctypes.byref(s), M, 16, 16,
                                                   ctypes.byref(ws), P(A16), P(A16), 0, P(0))
    for xt in (0, A16):
        for wt in (0, A16):
            s = F._Saved(A16, xt, A16, wt, A16, A16)
            assert fwd(s, 24) == ESHAPE
            for gt in (0, A16):
                assert bwd(s, F._BwdWs(A16, gt, A16), 24) == ESHAPE
            assert bwd(s, F._BwdWs(0, A16, A16), 16) == ENULL      # gy_q is required
    assert fwd(F._Saved(0, A16, A16, A16, A16, A16), 16) == ENULL  # x_q is required
    assert fwd(F._Saved(A16, MIS, A16, A16, A16, A16), 16) == EALIGN


def test_gemm_unscale_validation():
    g = lambda scale=A16, found=A16, C=A16B, M=16, fa=0: F.lib().fp8_gemm_unscale(
        P(A16), fa, P(A16B), 1, P(A16), P(A16), P(scale), P(found), P(C), M, 16, 32, P(0))
    assert g(scale=0) == ENULL and g(found=0) == ENULL and g(C=0) == ENULL
    assert g(M=24) == ESHAPE and g(fa=5) == EFORMAT
    assert g(C=MIS) == EALIGN and g(scale=A16 + 1) == EALIGN


def test_binding_refuses_a_missing_library(monkeypatch, tmp_path):
    # no fallback path: without the built library the binding raises
    monkeypatch.setattr(F, "_lib", None)
    monkeypatch.setattr(F, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        F.lib()


def test_size_limits():
    """Sizes beyond FP8SG_MAX_DIM / FP8SG_MAX_ELEMS are refused before any
    launch, products included (no int64 overflow on the way)."""
    text = open(HEADER).read()
    assert int(re.search(r"#define FP8SG_MAX_DIM \(1LL << (\d+)\)", text).group(1)) == 29 == \
        F.MAX_DIM.bit_length() - 1
    assert int(re.search(r"#define FP8SG_MAX_ELEMS \(1LL << (\d+)\)", text).group(1)) == 35 == \
        F.MAX_ELEMS.bit_length() - 1
    L = F.lib()
    D, E = F.MAX_DIM, F.MAX_ELEMS
    g = lambda M, N, K: L.fp8_gemm(P(A16), 0, P(A16B), 0, P(A16), P(A16), P(A16B), 0, M, N, K, P(0))
    assert g(D + 16, 16, 16) == ESHAPE and g(16, 16, D + 16) == ESHAPE
    assert g(1 << 20, 1 << 20, 16) == ESHAPE      # C has 2^40 elements
    assert g(1 << 62, 1 << 62, 1 << 62) == ESHAPE  # products that overflow int64
    assert L.fp8_amax(P(A16), E + 1, P(A16), P(0)) == ESHAPE
    assert L.fp8_quantize(P(A16), 1 << 20, 1 << 16, 0, P(A16), P(A16), P(0), P(0)) == ESHAPE
    assert L.fp8_quantize(P(A16), 1 << 62, 4, 0, P(A16), P(A16), P(0), P(0)) == ESHAPE
    rw = lambda r, c: L.fp8_quantize_rowwise(P(A16), r, c, 0, P(A16), P(A16), P(A16), P(0), P(0),
                                             P(0), P(0))
    assert rw(16, D + 16) == ESHAPE and rw(1 << 20, 1 << 20) == ESHAPE
    s = F._Saved(A16, A16, A16, A16, A16, A16)
    fwd = lambda M, N, K: L.fp8_scaled_linear_fwd(P(A16), P(A16), M, N, K, ctypes.byref(s), P(A16),
                                                  0, P(0))
    assert fwd(16, 16, D + 16) == ESHAPE and fwd(1 << 20, 1 << 20, 16) == ESHAPE
    ptrs = (ctypes.c_void_p * 1)(A16)
    numel = (ctypes.c_int64 * 1)(E + 1)
    assert L.amp_unscale_check(ptrs, numel, 1, P(A16), P(A16), P(0)) == ESHAPE
    assert L.amp_norm_workspace_len(numel, 1) == -1


def test_record_and_scalar_alignment():
    """Scale records and fp64 inverses need 8 bytes, fp32/int32 scalars 4."""
    L = F.lib()
    assert L.fp8_amax(P(A16), 16, P(A16 + 4), P(0)) == EALIGN
    assert L.fp8_quantize(P(A16), 4, 4, 0, P(A16 + 4), P(A16), P(0), P(0)) == EALIGN
    assert L.fp8_gemm(P(A16), 0, P(A16B), 0, P(A16 + 4), P(A16), P(A16B), 0, 16, 16, 16,
                      P(0)) == EALIGN
    s = F._Saved(A16, A16, A16, A16, A16 + 4, A16)
    assert L.fp8_scaled_linear_fwd(P(A16), P(A16), 16, 16, 16, ctypes.byref(s), P(A16), 0,
                                   P(0)) == EALIGN
    s = F._Saved(A16, A16, A16, A16, A16, A16)
    ws = F._BwdWs(A16, A16, A16 + 4)
    assert L.fp8_scaled_linear_bwd(P(A16), ctypes.byref(s), 16, 16, 16, ctypes.byref(ws), P(A16),
                                   P(A16), 0, P(0)) == EALIGN
    ptrs = (ctypes.c_void_p * 1)(A16)
    numel = (ctypes.c_int64 * 1)(8)
    assert L.amp_unscale_check(ptrs, numel, 1, P(A16 + 2), P(A16), P(0)) == EALIGN
    assert L.amp_unscale_check(ptrs, numel, 1, P(A16), P(A16 + 1), P(0)) == EALIGN
    for a in ((A16 + 2, A16, A16), (A16, A16 + 2, A16), (A16, A16, A16 + 1)):
        assert L.amp_update_scale(P(a[0]), P(a[1]), P(a[2]), 2.0, 0.5, 10, P(0)) == EALIGN


def test_binding_refuses_mismatched_buffers():
    """The library sees pointers only, so the binding checks dtype, shape,
    contiguity and device before any call (here on CPU tensors, which never
    reach the library)."""
    import torch
    u8, bf = torch.uint8, torch.bfloat16
    A = torch.zeros(32, 64, dtype=u8)
    B = torch.zeros(16, 64, dtype=u8)
    with pytest.raises(ValueError, match="shape"):
        F.fp8_gemm(A, 0, torch.zeros(16, 48, dtype=u8), 0, 0, 0, torch.zeros(32, 16, dtype=bf),
                   F.OUT_BF16)
    with pytest.raises(ValueError, match="shape"):
        F.fp8_gemm(A, 0, B, 0, 0, 0, torch.zeros(16, 32, dtype=bf), F.OUT_BF16)
    with pytest.raises(TypeError, match="dtype"):
        F.fp8_gemm(A, 0, B, 0, 0, 0, torch.zeros(32, 16, dtype=torch.float16), F.OUT_BF16)
    with pytest.raises(ValueError, match="contiguous"):
        F.fp8_gemm(A, 0, B, 0, 0, 0, torch.zeros(16, 32, dtype=bf).t(), F.OUT_BF16)
    with pytest.raises(ValueError, match="device"):
        F.fp8_gemm(A, 0, B, 0, 0, 0, torch.zeros(32, 16, dtype=bf), F.OUT_BF16)
    M, N, K = 32, 16, 64
    x, w = torch.zeros(M, K, dtype=bf), torch.zeros(N, K, dtype=bf)
    saved = F.LinearSaved(M, N, K, device="cpu")
    with pytest.raises(ValueError, match="shape"):
        F.fp8_scaled_linear_fwd(x, w, saved, torch.zeros(M, K, dtype=bf))
    with pytest.raises(ValueError, match="saved.x_qT"):
        F.fp8_scaled_linear_fwd(x, w, F.LinearSaved(M, N, K // 2, device="cpu",
                                                    tensors=(saved.x_q, saved.x_q.t().contiguous()[:K // 2],
                                                             saved.w_q, saved.w_qT, saved.recs)),
                                torch.zeros(M, N, dtype=bf))
    ws = F.LinearBwdWs(M, N + 16, device="cpu")
    with pytest.raises(ValueError, match="ws.gy_q"):
        F.fp8_scaled_linear_bwd(torch.zeros(M, N, dtype=bf), saved, ws, torch.zeros(M, K, dtype=bf),
                                torch.zeros(N, K, dtype=bf))
    with pytest.raises(TypeError, match="grads"):
        F.amp_unscale_check([torch.zeros(8, dtype=torch.float32)], torch.ones(1),
                            torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="history"):
        F.fp8_quantize_delayed(x, 0, F.ScaleRec(device="cpu"), torch.zeros(0),
                               torch.zeros(M, K, dtype=u8))
    rs = F.RowScalesDev(M, device="cpu")
    with pytest.raises(ValueError, match="cols_sc.amax"):
        F.fp8_quantize_rowwise(x, 0, rs, torch.zeros(M, K, dtype=u8), F.RowScalesDev(K - 16, device="cpu"),
                               torch.zeros(K, M, dtype=u8))


def test_delayed_and_rowwise_fused_unscale_validation():
    L = F.lib()
    s = F._Saved(A16, A16, A16, A16, A16, A16)
    ws = F._BwdWs(A16, A16, A16)
    d = lambda hist=A16, h=4, scale=A16, found=A16, M=16: L.fp8_scaled_linear_bwd_delayed_unscale(
        P(A16), ctypes.byref(s), M, 16, 16, ctypes.byref(ws), P(hist), h, P(scale), P(found),
        P(A16), P(A16), P(0))
    assert d(hist=0) == ENULL and d(scale=0) == ENULL and d(found=0) == ENULL
    assert d(h=0) == ESHAPE and d(M=8) == ESHAPE
    assert d(hist=A16 + 2) == EALIGN and d(scale=A16 + 2) == EALIGN and d(found=A16 + 1) == EALIGN
    srw = F._SavedRW(*([A16] * 12))
    wrw = F._BwdWsRW(*([A16] * 6))
    r = lambda scale=A16, found=A16, gx=A16, M=16: L.fp8_scaled_linear_bwd_rowwise_unscale(
        P(A16), ctypes.byref(srw), M, 16, 32, ctypes.byref(wrw), P(scale), P(found), P(gx),
        P(A16), P(0))
    assert r(scale=0) == ENULL and r(found=0) == ENULL and r(gx=0) == ENULL
    assert r(M=24) == ESHAPE and r(M=0) == ESHAPE
    assert r(scale=A16 + 1) == EALIGN and r(gx=MIS) == EALIGN


def test_buffer_checks_are_cached_per_buffer_set():
    """A LinearSaved/LinearBwdWs validated once is not re-checked while its
    buffers and sizes stay the same, and is checked again when one changes."""
    import torch
    M, N, K = 32, 16, 64
    saved = F.LinearSaved(M, N, K, device="cpu")
    saved.check(M, N, K)
    saved.check(M, N, K)  # cached
    saved.x_q = torch.zeros(M, K + 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="saved.x_q"):
        saved.check(M, N, K)
    saved.x_q = torch.zeros(M, K, dtype=torch.uint8)
    saved.check(M, N, K)
    with pytest.raises(ValueError, match="saved.x_q"):
        saved.check(M, N, K + 16)  # other sizes: checked again
    ws = F.LinearBwdWs(M, N, device="cpu")
    ws.check(M, N)
    ws.gy_qT = torch.zeros(N, M, dtype=torch.int8)
    with pytest.raises(TypeError, match="ws.gy_qT"):
        ws.check(M, N)


def test_linear_copies_query():
    """fp8_linear_copies validates like a linear layer's entry points and
    never asks for W's copy (host-only: no launch)."""
    L = F.lib()
    v = [ctypes.c_int32(7) for _ in range(3)]
    q = lambda M, N, K, ptrs=None: L.fp8_linear_copies(M, N, K, *(ptrs or [ctypes.addressof(a) for a in v]))
    assert q(64, 256, 24) == ESHAPE and q(0, 256, 128) == ESHAPE and q(-16, 16, 16) == ESHAPE
    assert q(64, 256, 128, [0, ctypes.addressof(v[1]), ctypes.addressof(v[2])]) == ENULL
    for shape in ((64, 256, 128), (8192, 14336, 4096), (8192, 4096, 14336), (4096, 4096, 4096)):
        assert q(*shape) == 0
        assert v[1].value == 0 and v[0].value in (0, 1) and v[2].value in (0, 1)
        assert not (v[0].value and v[2].value)
        assert F.fp8_linear_copies(*shape) == tuple(bool(a.value) for a in v)
