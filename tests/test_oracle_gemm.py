"""Pins for the oracle GEMM C = (A . B^T) * fl32(inv_a * inv_b), fp32 accumulation
[AMP-MP "不要忘记 Accumulator Precision"; FP8-TRAIN §2, §4].

Every e4m3 value is an integer times 2^-9 and every e5m2 value an integer
times 2^-16, so the exact dot product is an integer times 2^-18 (e4m3 x e4m3)
or 2^-25 (e5m2 x e4m3): Python integers give it with no rounding at all.  The
oracle's fp32 result must then lie inside the textbook bound for recursive
summation, |fl(sum) - sum| <= gamma_K * sum|a_k b_k| with gamma_K = K u/(1-K u),
u = 2^-24, plus one rounding of the final scaling.  A transposed operand, a
wrong index or a dropped term breaks the bound by orders of magnitude.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

UNIT = {O.E4M3FN: 9, O.E5M2: 16}  # value = integer * 2^-UNIT
U = 2.0 ** -24


def int_codes(fmt, codes):
    """Exact integer numerators of the codes' values (finite codes only)."""
    v = O.decode(fmt, codes)
    n = v * 2.0 ** UNIT[fmt]
    assert np.all(n == np.round(n))
    return n.astype(np.int64)


def random_codes(rng, fmt, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    bad = np.isnan(O.decode(fmt, c)) | np.isinf(O.decode(fmt, c))
    c[bad] = 0x00
    return c


@pytest.mark.parametrize("fa,fb,M,N,K", [
    (O.E4M3FN, O.E4M3FN, 7, 5, 64),
    (O.E5M2, O.E4M3FN, 6, 9, 128),
    (O.E4M3FN, O.E4M3FN, 3, 4, 1000),
    (O.E5M2, O.E4M3FN, 5, 3, 257),
])
def test_gemm_exact_integer_bound(fa, fb, M, N, K):
    rng = np.random.default_rng(M * 1000 + K)
    A = random_codes(rng, fa, (M, K))
    B = random_codes(rng, fb, (N, K))
    inv_a, inv_b = 0.37, 2.0 ** -5
    C = O.gemm(A, fa, B, fb, inv_a, inv_b)
    alpha = float(O.gemm_alpha(inv_a, inv_b))
    ia, ib = int_codes(fa, A), int_codes(fb, B)
    den = 2 ** (UNIT[fa] + UNIT[fb])
    gam = K * U / (1 - K * U)
    for i in range(M):
        for j in range(N):
            exact = Fraction(int(sum(int(x) * int(y) for x, y in zip(ia[i], ib[j]))), den)
            absum = Fraction(int(sum(abs(int(x) * int(y)) for x, y in zip(ia[i], ib[j]))), den)
            # acc error (recursive summation) then one rounding of acc*alpha
            acc_bound = gam * float(absum)
            ref = float(exact) * alpha
            bound = acc_bound * alpha + U * (abs(ref) + acc_bound * alpha) + 1e-45
            assert abs(float(C[i, j]) - ref) <= bound, (i, j, C[i, j], ref, bound)


def test_gemm_exact_when_partial_sums_are_representable():
    # small-integer operands: every partial sum is an integer < 2^24, so fp32 accumulation
    # is exact, and alpha a power of two keeps the scaling exact
    rng = np.random.default_rng(5)
    vals = np.arange(-8, 9, dtype=np.float64)
    A = O.encode(O.E4M3FN, rng.choice(vals, (12, 96)))
    B = O.encode(O.E4M3FN, rng.choice(vals, (10, 96)))
    Ad = O.decode(O.E4M3FN, A)
    Bd = O.decode(O.E4M3FN, B)
    C = O.gemm(A, O.E4M3FN, B, O.E4M3FN, 2.0 ** -3, 2.0 ** 7)
    assert np.array_equal(C, ((Ad @ Bd.T) * 16.0).astype(np.float32))
    # not symmetric in the operands' roles: C^T comes from swapping them
    Ct = O.gemm(B, O.E4M3FN, A, O.E4M3FN, 2.0 ** -3, 2.0 ** 7)
    assert np.array_equal(Ct, C.T)


def test_gemm_closed_forms():
    one = O.encode(O.E4M3FN, [1.0])[0]
    zero = np.uint8(0)
    K = 64
    rng = np.random.default_rng(9)
    B = random_codes(rng, O.E5M2, (K, K))  # any e5m2 values
    # A = a row-selection (permutation) matrix of ones: C rows are rows of B^T ... i.e.
    # C[i, j] = sum_k P[i,k] B[j,k] = B[j, p(i)]
    perm = rng.permutation(K)
    P = np.full((K, K), zero, np.uint8)
    P[np.arange(K), perm] = one
    C = O.gemm(B, O.E5M2, P, O.E4M3FN, 1.0, 1.0)  # C[i, j] = B[i, perm[j]]
    assert np.array_equal(C, O.decode(O.E5M2, B)[:, perm].astype(np.float32))
    # rank one, all equal: C = K * a * b exactly
    a = O.encode(O.E5M2, [0.75])[0]
    b = O.encode(O.E4M3FN, [-3.5])[0]
    A = np.full((3, K), a, np.uint8)
    Bm = np.full((4, K), b, np.uint8)
    C = O.gemm(A, O.E5M2, Bm, O.E4M3FN, 0.5, 4.0)
    assert np.all(C == np.float32(K * 0.75 * -3.5 * 2.0))


def test_gemm_sampled_matches_full():
    rng = np.random.default_rng(3)
    A = random_codes(rng, O.E5M2, (33, 80))
    B = random_codes(rng, O.E4M3FN, (17, 80))
    C = O.gemm(A, O.E5M2, B, O.E4M3FN, 0.1, 0.3)
    ii = rng.integers(0, 33, 50)
    jj = rng.integers(0, 17, 50)
    assert np.array_equal(O.gemm_at(A, O.E5M2, B, O.E4M3FN, 0.1, 0.3, ii, jj), C[ii, jj])
    mag = O.gemm_absdot_at(A, O.E5M2, B, O.E4M3FN, 0.1, 0.3, ii, jj)
    Ad, Bd = O.decode(O.E5M2, A), O.decode(O.E4M3FN, B)
    ref = (np.abs(Ad)[ii] * np.abs(Bd)[jj]).sum(1) * float(O.gemm_alpha(0.1, 0.3))
    assert np.allclose(mag, ref, rtol=1e-12)


def test_linear_composition_shapes_and_roles():
    """fwd x@W^T, dgrad gy@W, wgrad gy^T@x [FP8-TRAIN §4], checked against fp64
    products of the dequantised codes."""
    import workloads as W
    x = W.normal_bf16(21, 1, (32, 48), 1.0)
    w = W.normal_bf16(21, 2, (40, 48), 0.02)
    gy = W.normal_bf16(21, 3, (32, 40), 1e-3)
    fw = O.linear_fwd(x, w)
    bw = O.linear_bwd(gy, fw)
    xd = O.decode(O.E4M3FN, fw.x.q) * fw.x.sc.inv
    wd = O.decode(O.E4M3FN, fw.w.q) * fw.w.sc.inv
    gd = O.decode(O.E5M2, bw.gy.q) * bw.gy.sc.inv
    for got, ref in ((fw.c, xd @ wd.T), (bw.c_gx, gd @ wd), (bw.c_gw, gd.T @ xd)):
        assert got.shape == ref.shape
        assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    # outputs are the bf16 rounding of the fp32 results
    assert np.array_equal(fw.y, O.encode(O.BF16, fw.c))
