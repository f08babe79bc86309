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


def round_binary(x: Fraction, p: int, emin: int) -> Fraction:
    """x rounded to the nearest binary floating-point number with p significant
    bits and smallest normal exponent emin, ties to even (IEEE 754
    roundTiesToEven; no overflow handling: the values here stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    ulp = Fraction(2) ** (max(e, emin) - (p - 1))
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def fl64(x: Fraction) -> Fraction:
    return round_binary(x, 53, -1022)


def fl32(x: Fraction) -> Fraction:
    return round_binary(x, 24, -126)


def alpha_reading(inv_a: float, inv_b: float) -> float:
    """The epilogue factor as read from FP8-TRAIN §2 (dequantise by the product of
    the two inverse scales): the fp64 product of the two fp64 inverses, rounded
    to fp32 -- here from the exact rational product, two roundings by hand."""
    return float(fl32(fl64(Fraction(inv_a) * Fraction(inv_b))))


def test_round_binary_against_hardware_casts():
    # the hand rounding agrees with numpy's IEEE casts on random doubles
    rng = np.random.default_rng(17)
    for v in np.exp(rng.uniform(-60.0, 60.0, 2000)) * rng.choice([-1.0, 1.0], 2000):
        assert float(fl32(Fraction(float(v)))) == float(np.float32(v))
    for a, b in rng.uniform(-1e3, 1e3, (500, 2)):
        assert float(fl64(Fraction(float(a)) * Fraction(float(b)))) == float(a) * float(b)


def inverse_pairs(n, seed):
    """Inverse scales as the quantizer makes them, inv = 1 / (fp8_max / amax),
    from amax values across the workloads' range."""
    rng = np.random.default_rng(seed)
    amax = np.exp(rng.uniform(np.log(1e-6), np.log(1e4), (n, 2)))
    fmax = np.array([448.0, 57344.0])
    return 1.0 / (fmax / amax)


def test_gemm_alpha_is_rounded_fp64_product():
    """orc_gemm_alpha = fl32(fl64(inv_a * inv_b)), checked against exact rational
    arithmetic on pairs where the other plausible reading, fl32(fl32(inv_a) *
    fl32(inv_b)) (rounding each inverse to fp32 first), gives a different value:
    a swapped rounding order fails here."""
    differ = 0
    for inv_a, inv_b in inverse_pairs(4000, 23):
        inv_a, inv_b = float(inv_a), float(inv_b)
        ref = alpha_reading(inv_a, inv_b)
        assert float(O.gemm_alpha(inv_a, inv_b)) == ref, (inv_a, inv_b)
        alt = float(fl32(fl32(Fraction(inv_a)) * fl32(Fraction(inv_b))))
        differ += alt != ref
        # the single correct rounding of the exact product: the same value
        # unless the fp64 step lands on an fp32 midpoint (never for these pairs)
        assert float(fl32(Fraction(inv_a) * Fraction(inv_b))) == ref
    assert differ > 500  # the pin separates the readings on many pairs


def test_gemm_alpha_double_rounding_case():
    """A product whose fp64 rounding lands exactly on an fp32 midpoint: the exact
    product of these two doubles lies just above 1 + 2^-24, the midpoint between
    1 and 1 + 2^-23, and within half an fp64 ulp of it, so its fp64 rounding is
    the midpoint and ties to even give 1.0; rounding the exact product once would
    give 1 + 2^-23.  The reading (fp64 product, then fp32) decides this case."""
    a, b = 1.3184808436607272, 0.7584486831285095
    mid = Fraction(1) + Fraction(1, 2 ** 24)
    exact = Fraction(a) * Fraction(b)
    assert mid < exact < mid + Fraction(1, 2 ** 53)
    assert float(O.gemm_alpha(a, b)) == alpha_reading(a, b) == 1.0
    assert float(fl32(exact)) == 1.0 + 2.0 ** -23


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
    # inverses that are not powers of two, so the epilogue factor's rounding
    # matters; alpha comes from exact arithmetic, not from the oracle
    inv_a, inv_b = 0.37, 1.0 / (448.0 / 3.3)
    C = O.gemm(A, fa, B, fb, inv_a, inv_b)
    alpha = alpha_reading(inv_a, inv_b)
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
