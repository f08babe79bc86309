"""Comparison helpers shared by the GPU parity tests, the smoke check and the
benchmark's sampled checks.  They compare HIP results with oracle results; they
compute nothing of the method themselves beyond the error bound.

GEMM tolerance.  Both the HIP kernel and the oracle accumulate exact FP8
products in fp32, in different orders.  For recursive summation of K terms
|fl(s) - s| <= gamma_K * sum|a_k b_k|, gamma_K = K u / (1 - K u), u = 2^-24,
for any order, so two fp32 results differ by at most 2 gamma_K sum|a_k b_k|;
scaling by alpha adds one rounding each.  That is the elementwise bound used
for fp32 outputs; bf16/fp16 outputs may in addition sit one unit in the last
place of the output format away.  The normwise figure
max|C_gpu - C_ref| / max|C_ref| must also stay within 1e-3.
"""
import numpy as np

import oracle as O

U32 = 2.0 ** -24
NORMWISE_TOL = 1e-3


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
    bound = 2.0 * gamma(K) * absdot + 2.0 * U32 * np.abs(c_ref) + 1e-38
    if out_fmt is not None:
        bound = bound + ulp_at(out_fmt, c_ref)
    err = np.abs(got - c_ref)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, f"{what}: {bad.size} outputs outside the bound, first {bad[:4]}: " \
                          f"got {got[bad[:4]]} ref {c_ref[bad[:4]]} bound {bound[bad[:4]]}"
    scale = np.abs(c_ref).max() if c_ref.size else 0.0
    if scale > 0:
        nw = err.max() / scale
        assert nw <= NORMWISE_TOL, f"{what}: normwise error {nw}"
        return nw
    return 0.0


def decode_out(out_fmt, arr):
    if out_fmt is None:
        return np.asarray(arr, np.float64)
    return O.decode(out_fmt, arr)
