"""Pins for the oracle's codecs (fp8 e4m3fn / e5m2, fp16, bf16).

The oracle is checked against what the pages print (maxima, field widths,
levels per octave, the worked rounding examples) and against independent
encoders: torch's CPU casts for the FP8 formats and bf16, numpy's for fp16.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from conftest import golden

FMT_NAMES = {O.E4M3FN: "e4m3fn", O.E5M2: "e5m2", O.F16: "fp16", O.BF16: "bf16"}
TORCH_DT = {O.E4M3FN: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2, O.BF16: torch.bfloat16}


def all_codes(fmt):
    n = 256 if fmt in O.FP8_FORMATS else 65536
    return np.arange(n, dtype=O.code_dtype(fmt))


def fields(code, e, m):
    return code >> (e + m), (code >> m) & ((1 << e) - 1), code & ((1 << m) - 1)


def lib_encode(fmt, v32):
    """Independent encoder: torch CPU cast (FP8, bf16) or numpy cast (fp16)."""
    v32 = np.ascontiguousarray(v32, np.float32)
    if fmt == O.F16:
        with np.errstate(over="ignore"):
            return v32.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(v32).to(TORCH_DT[fmt])
    if fmt == O.BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def is_nan_code(fmt, codes):
    return np.isnan(O.decode(fmt, codes))


# ------------------------------------------------------------- printed facts

def test_printed_maxima_and_layouts():
    g = golden("formats.json")
    assert O.fp8_max(O.E4M3FN) == g["e4m3fn"]["max"] == 448.0
    assert O.fp8_max(O.E5M2) == g["e5m2"]["max"] == 57344.0
    # largest finite codes and their fields: S.EEEE.MMM = 0.1111.110, S.EEEEE.MM = 0.11110.11
    assert O.max_code(O.E4M3FN) == 0x7E and fields(0x7E, 4, 3) == (0, 0b1111, 0b110)
    assert O.max_code(O.E5M2) == 0x7B and fields(0x7B, 5, 2) == (0, 0b11110, 0b11)
    # 448 = 1.75 * 2^8 and 57344 = 1.75 * 2^15: biases 7 and 15
    assert O.decode(O.E4M3FN, [0x7E])[0] == 1.75 * 2 ** (0b1111 - 7)
    assert O.decode(O.E5M2, [0x7B])[0] == 1.75 * 2 ** (0b11110 - 15)
    assert O.decode(O.F16, [0x7BFF])[0] == g["fp16"]["max"]
    # fp16 smallest normal 2^-14 ~ 6.1e-5
    mn = O.decode(O.F16, [0x0400])[0]
    assert mn == 2.0 ** -14 and abs(mn - g["fp16"]["min_normal_approx"]) < 1e-6
    bmax = O.decode(O.BF16, [0x7F7F])[0]
    assert math.isclose(bmax, g["bf16"]["max_approx"], rel_tol=0.01)
    assert math.isclose(O.decode(O.BF16, [0x0080])[0], g["bf16"]["min_normal_approx"], rel_tol=0.05)  # printed to 2 digits


@pytest.mark.parametrize("fmt,n_nan,n_inf,min_sub", [
    (O.E4M3FN, 2, 0, 2.0 ** -9),
    (O.E5M2, 6, 2, 2.0 ** -16),
])
def test_exhaustive_fp8_census(fmt, n_nan, n_inf, min_sub):
    v = O.decode(fmt, all_codes(fmt))
    assert np.isnan(v).sum() == n_nan
    assert np.isinf(v).sum() == n_inf
    fin = v[np.isfinite(v)]
    assert fin.max() == O.fp8_max(fmt) and fin.min() == -O.fp8_max(fmt)
    assert np.min(np.abs(fin[fin != 0])) == min_sub
    # +0 and -0 only
    assert np.sum(fin == 0) == 2
    assert np.signbit(v[0x80]) and v[0x80] == 0


@pytest.mark.parametrize("fmt,levels", [(O.E4M3FN, 8), (O.E5M2, 4), (O.F16, 1024), (O.BF16, 128)])
def test_levels_per_octave(fmt, levels):
    # e4m3 has 8 mantissa levels per octave [FP8-TRAIN §3 table]; every normal binade
    # [2^e, 2^(e+1)) holds 2^mbits codes.
    if fmt == O.E4M3FN:
        assert golden("formats.json")["e4m3fn"]["levels_per_octave"] == levels
    v = O.decode(fmt, np.arange(O.max_code(fmt) + 1))
    normal = v[v >= v[1 << int(math.log2(levels))]]  # from the smallest normal upward
    e = np.floor(np.log2(normal)).astype(int)
    counts = np.bincount(e - e.min())
    assert np.all(counts[:-1] == levels)
    assert counts[-1] <= levels  # top binade (e4m3fn loses its NaN pattern there)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2, O.F16, O.BF16])
def test_roundtrip_and_monotonic(fmt):
    c = all_codes(fmt)
    v = O.decode(fmt, c)
    ok = ~np.isnan(v)
    assert np.array_equal(O.encode(fmt, v[ok]), c[ok])
    pos = v[: O.max_code(fmt) + 1]
    assert np.all(np.diff(pos) > 0)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2, O.F16, O.BF16])
def test_midpoints_round_to_even(fmt):
    mc = O.max_code(fmt)
    c = np.arange(mc, dtype=np.int64)
    v = O.decode(fmt, c)
    vn = O.decode(fmt, c + 1)
    mid = 0.5 * (v + vn)
    got = O.encode(fmt, mid).astype(np.int64)
    even = np.where(c % 2 == 0, c, c + 1)
    assert np.array_equal(got, even)
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(O.encode(fmt, below).astype(np.int64), c)
    assert np.array_equal(O.encode(fmt, above).astype(np.int64), c + 1)


def test_overflow_and_specials():
    # e4m3fn has no inf: past the top grid step -> NaN; e5m2 / fp16 -> inf
    assert O.encode(O.E4M3FN, [464.0])[0] == 0x7E  # tie with the (reserved) next step -> even
    assert O.encode(O.E4M3FN, [465.0, np.inf])[0] == 0x7F
    assert O.encode(O.E5M2, [61439.0])[0] == 0x7B
    assert O.encode(O.E5M2, [61440.0, np.inf])[0] == 0x7C
    assert O.encode(O.F16, [65519.0])[0] == 0x7BFF and O.encode(O.F16, [65520.0])[0] == 0x7C00
    assert O.encode(O.E4M3FN, [-0.0])[0] == 0x80 and O.encode(O.E5M2, [-1e-30])[0] == 0x80
    assert all(is_nan_code(f, O.encode(f, [np.nan])) for f in (O.E4M3FN, O.E5M2, O.F16, O.BF16))


# ------------------------------------------- independent encoders (torch, numpy)

def sweep_values(fmt, n_random, seed):
    rng = np.random.default_rng(seed)
    mc = O.max_code(fmt)
    v = O.decode(fmt, np.arange(mc + 1))
    vn = np.append(v[1:], 2 * v[-1] - v[-2])
    mid = (0.5 * (v + vn)).astype(np.float32)  # exact in fp32 for every format here
    pts = [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf)),
           v.astype(np.float32)]
    top = float(vn[-1]) * 1.5
    lo = float(v[1]) / 8
    with np.errstate(over="ignore"):
        mags = np.exp(rng.uniform(np.log(lo), np.log(top), n_random)).astype(np.float32)
    pts.append(mags)
    # random fp32 bit patterns of moderate magnitude
    bits = rng.integers(0, 0x7F800000, n_random, dtype=np.int64).astype(np.uint32)
    pts.append(bits.view(np.float32))
    allp = np.concatenate(pts)
    allp = allp[np.isfinite(allp)]
    return np.concatenate([allp, -allp])


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2, O.F16, O.BF16])
def test_encoder_matches_library_casts(fmt):
    vals = sweep_values(fmt, 400_000, 1234 + fmt)
    mine = O.encode(fmt, vals)
    ref = lib_encode(fmt, vals)
    nan_m, nan_r = is_nan_code(fmt, mine), is_nan_code(fmt, ref)
    assert np.array_equal(nan_m, nan_r)
    bad = np.nonzero((mine != ref) & ~nan_m)[0]
    assert bad.size == 0, [(float(vals[i]), hex(mine[i]), hex(ref[i])) for i in bad[:8]]


def test_fp16_spacing_example():
    g = golden("fp16_spacing.json")
    one = O.encode(O.F16, np.float32([g["w"]]))
    upd = np.float32(O.decode(O.F16, one)[0]) + np.float32(g["update"])
    assert O.decode(O.F16, O.encode(O.F16, np.float32([upd])))[0] == g["result"]
    sp = O.decode(O.F16, [0x3C01])[0] - 1.0  # spacing just above 1.0
    assert abs(sp - g["spacing_approx"]) < 2.5e-5


def test_bf16_master_weight_example():
    g = golden("bf16_master_weight.json")
    w_bf16 = O.encode(O.BF16, np.float32([g["w0"]]))[0]
    w_next = O.decode(O.BF16, [w_bf16 - 1])[0]
    assert w_next == g["next_down"] and g["w0"] - w_next == g["bf16_spacing"]
    master = np.float32(g["w0"])
    direct = w_bf16
    first = None
    for step in range(1, 8):
        master = np.float32(master + np.float32(g["delta"]))
        cast = O.decode(O.BF16, O.encode(O.BF16, np.float32([master])))[0]
        d = np.float32(O.decode(O.BF16, [direct])[0]) + np.float32(g["delta"])
        direct = O.encode(O.BF16, np.float32([d]))[0]
        assert O.decode(O.BF16, [direct])[0] == g["w0"]  # the bf16-stored weight never moves
        if first is None and cast != g["w0"]:
            first = step
            assert cast == g["next_down"]
    assert first == g["first_change_step"]
