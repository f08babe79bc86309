"""Pins for the oracle's global gradient norm (sum of squares of the unscaled
fp16 gradients taken together, the quantity gradient clipping uses after
unscale ["AMP：Automatic Mixed Precision 技术笔记", §6 gradient clipping; "06 ·
混合精度", §四]).  The oracle sums exactly in 128-bit integers; the pins check
it against an independent decoder (numpy's float16) with exact rational
arithmetic, closed forms, and the multi-tensor definition."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def exact_by_fractions(arrays):
    tot = Fraction(0)
    for a in arrays:
        for v in a.view(np.float16).astype(np.float64):
            tot += Fraction(float(v)) ** 2
    return tot


def rand_f16(seed, n, lo=-30, hi=15):
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(lo, hi, n)
    v = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float16)
    v[~np.isfinite(v)] = np.float16(1.0)
    return v.view(np.uint16).copy()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_exact_against_fractions(seed):
    a = rand_f16(seed, 300)
    b = rand_f16(seed + 10, 77, lo=-24, hi=-14)  # fp16 subnormals and the normal edge
    kind, total = O.sumsq_f16([a, b])
    assert kind == 0
    assert Fraction(total, 2 ** 48) == exact_by_fractions([a, b])


def test_closed_forms():
    one = np.full(1000, 0x3C00, np.uint16)           # 1.0
    assert O.sumsq_f16([one]) == (0, 1000 * 2 ** 48)
    mx = np.full(7, 0x7BFF, np.uint16)               # 65504, the fp16 maximum
    assert O.sumsq_f16([mx]) == (0, 7 * 65504 ** 2 * 2 ** 48)
    tiny = np.full(5, 0x0001, np.uint16)             # 2^-24, the smallest subnormal
    assert O.sumsq_f16([tiny]) == (0, 5)
    zero = np.array([0x0000, 0x8000], np.uint16)     # +0 and -0
    assert O.sumsq_f16([zero]) == (0, 0)
    neg = one | np.uint16(0x8000)                    # -1.0: the sign does not matter
    assert O.sumsq_f16([neg]) == O.sumsq_f16([one])
    s, nrm = O.grad_norm([np.full(16, 0x4400, np.uint16)])  # sixteen 4.0 -> 256, norm 16
    assert (s, nrm) == (256.0, 16.0)


def test_split_into_tensors_is_the_same_sum():
    a = rand_f16(7, 10_000)
    whole = O.sumsq_f16([a])
    parts = O.sumsq_f16([a[:1], a[1:4097], a[4097:9999], a[9999:]])
    assert whole == parts


def test_nonfinite_kinds():
    a = rand_f16(8, 100)
    inf = a.copy(); inf[17] = 0x7C00
    ninf = a.copy(); ninf[3] = 0xFC00
    nan = a.copy(); nan[50] = 0x7E00
    assert O.sumsq_f16([inf])[0] == 1 and O.sumsq_f16([ninf])[0] == 1
    assert O.sumsq_f16([nan])[0] == 2 and O.sumsq_f16([inf, nan])[0] == 2
    assert O.grad_norm([inf]) == (math.inf, math.inf)
    assert all(math.isnan(v) for v in O.grad_norm([a, nan]))


def test_against_float64_sum():
    a = rand_f16(9, 200_000, lo=-20, hi=8)
    s, nrm = O.grad_norm([a])
    v = a.view(np.float16).astype(np.float64)
    ref = float(np.sum(v * v))  # every square is exact in float64; only the sum rounds
    assert abs(s - ref) <= a.size * 2.0 ** -53 * ref
    assert nrm == math.sqrt(s)
