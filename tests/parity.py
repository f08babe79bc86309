"""Comparison helpers shared by the GPU parity tests, the smoke check and the
benchmark's sampled checks.  They compare HIP results with oracle results; they
compute nothing of the method themselves beyond the error bound.

GEMM tolerance.  The oracle sums the exact FP8 products in fp32, in k order.
The gfx950 FP8 matrix instruction (v_mfma_f32_16x16x128_f8f6f4) also forms
every product exactly, but adds each group of 8 products with a narrow
alignment window before the fp32 accumulation: measured on the device, a
product 2^-14 or more below the group's largest one is dropped, one 2^-13
below is kept.  So within a group of 8 every product other than the largest
loses less than 2^-13 of the largest, i.e. the group sum is off by less than
7 * 2^-13 * max|p| <= 2^-10 * sum_group |p|.  The fp32 accumulation of the
group sums and the oracle's sequential fp32 sum each add at most
gamma_K * sum|p| (gamma_K = K u / (1 - K u), u = 2^-24), and the scaling by
alpha one rounding each.  Elementwise bound:
    |C_gpu - C_ref| <= (2^-10 + 2 gamma_K) * sum_k |a_k b_k| * |alpha| + 2u |C_ref|
which is also within the required 1e-3 relative error measured against the
magnitude sum_k |a_k b_k| |alpha| of the dot product (the measure that stays
meaningful where the terms cancel).  bf16/fp16 outputs may in addition sit one
unit in the last place of the output format away.  For fp32 outputs the
normwise figure max|C_gpu - C_ref| / max|C_ref| must stay within 1e-3 too.
"""
import numpy as np

import oracle as O

U32 = 2.0 ** -24
NORMWISE_TOL = 1e-3
GROUP_ALIGN = 2.0 ** -10  # 7 * 2^-13, rounded up: the matrix instruction's 8-product groups


def gamma(k: int) -> float:
    return k * U32 / (1.0 - k * U32)


def assert_codes_equal(fmt, got, ref, what=""):
    """Bit-exact codes, except that where the oracle writes NaN any NaN code of
    the format is accepted (several NaN encodings are correct)."""
    got = np.asarray(got).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    assert got.shape == ref.shape, what
    nan_ref = np.isnan(O.decode(fmt, ref))
    nan_got = np.isnan(O.decode(fmt, got))
    assert np.array_equal(nan_ref, nan_got), f"{what}: NaN positions differ"
    bad = np.nonzero((got != ref) & ~nan_ref)[0]
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[:5]}: " \
                          f"got {[hex(int(got[i])) for i in bad[:5]]} ref {[hex(int(ref[i])) for i in bad[:5]]}"


def ulp_at(out_fmt, c_ref):
    """Spacing of the output format at each reference value."""
    code = O.encode(out_fmt, np.asarray(c_ref, np.float32)).astype(np.int64)
    mag = code & 0x7FFF
    lo = O.decode(out_fmt, mag.astype(np.uint16))
    hi = O.decode(out_fmt, np.minimum(mag + 1, 0x7BFF if out_fmt == O.F16 else 0x7F7F).astype(np.uint16))
    return np.abs(hi - lo)


def check_gemm_values(got, c_ref, absdot, K, out_fmt=None, what=""):
    """got: fp32 values (or decoded bf16/fp16 values) of the GPU output at the
    same positions as c_ref (oracle fp32) and absdot (sum|a b| * |alpha|)."""
    got = np.asarray(got, np.float64).reshape(-1)
    c_ref = np.asarray(c_ref, np.float64).reshape(-1)
    absdot = np.asarray(absdot, np.float64).reshape(-1)
    bound = (GROUP_ALIGN + 2.0 * gamma(K)) * absdot + 2.0 * U32 * np.abs(c_ref) + 1e-38
    if out_fmt is not None:
        bound = bound + ulp_at(out_fmt, c_ref)
    err = np.abs(got - c_ref)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, f"{what}: {bad.size} outputs outside the bound, first {bad[:4]}: " \
                          f"got {got[bad[:4]]} ref {c_ref[bad[:4]]} bound {bound[bad[:4]]}"
    scale = np.abs(c_ref).max() if c_ref.size else 0.0
    nw = err.max() / scale if scale > 0 else 0.0
    if out_fmt is None:
        # the required 1e-3 relative error, elementwise against the dot product's
        # magnitude and normwise against the largest output
        rel = err / np.maximum(absdot, 1e-38)
        assert np.all(rel <= NORMWISE_TOL), f"{what}: relative error {rel.max()}"
        if scale > 0:
            assert nw <= NORMWISE_TOL, f"{what}: normwise error {nw}"
    return nw


def decode_out(out_fmt, arr):
    if out_fmt is None:
        return np.asarray(arr, np.float64)
    return O.decode(out_fmt, arr)


def check_unscaled_values(got_f16, c_ref, absdot, K, loss_scale, what=""):
    """fp16 gradients unscaled in a GEMM epilogue, g = fp16(fl32(h) / S) with
    h = fp16(c) and a power-of-two loss scale S, against the oracle's GEMM value
    c (fp32, before the unscale): S * g is h exactly unless g is an fp16
    subnormal (then within S * 2^-25).  Bound: the summation bound above, one
    fp16 ulp of the value, and that subnormal step."""
    got = np.asarray(decode_out(O.F16, got_f16), np.float64).reshape(-1) * loss_scale
    c_ref = np.asarray(c_ref, np.float64).reshape(-1)
    absdot = np.asarray(absdot, np.float64).reshape(-1)
    err = np.abs(got - c_ref)
    bound = ((GROUP_ALIGN + 2.0 * gamma(K)) * absdot + 2.0 * U32 * np.abs(c_ref)
             + ulp_at(O.F16, c_ref) + loss_scale * 2.0 ** -25)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, f"{what}: {bad.size} unscaled values outside the bound, first {bad[:4]}"
    scale = np.abs(c_ref).max() if c_ref.size else 0.0
    return float(err.max() / scale) if scale > 0 else 0.0
