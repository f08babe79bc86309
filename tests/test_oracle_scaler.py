"""Pins for the oracle's GradScaler step: unscale, non-finite check and the
update() state machine [PT-CH20 §20.2.2, §20.5.33; AMP-NOTES §4; MP-06 §四]."""
import numpy as np
import pytest

import oracle as O
from conftest import golden


def run(found_seq, interval, init=65536.0, growth=2.0, backoff=0.5):
    st = O.ScalerState(np.float32(init), 0)
    out = []
    for f in found_seq:
        st = O.update_scale(st, f, growth, backoff, interval)
        out.append((float(st.scale), st.tracker))
    return out


def test_defaults_are_the_pages():
    g = golden("gradscaler.json")
    assert (g["init_scale"], g["growth_factor"], g["backoff_factor"], g["growth_interval"]) == \
        (2.0 ** 16, 2.0, 0.5, 2000)


@pytest.mark.parametrize("interval,n", [(1, 20), (3, 50), (100, 1000), (2000, 4500)])
def test_closed_form_without_overflow(interval, n):
    # no inf/NaN: scale_n = init * growth^floor(n/I), tracker_n = n mod I
    traj = run([0] * n, interval)
    for k, (s, t) in enumerate(traj, start=1):
        assert s == 65536.0 * 2.0 ** (k // interval)
        assert t == k % interval


def test_brute_force_short_sequence():
    # I = 3 over clean, clean, clean, inf, clean: x2 at step 3, x0.5 at step 4
    assert run([0, 0, 0, 1, 0], 3) == [(65536.0, 1), (65536.0, 2), (131072.0, 0),
                                        (65536.0, 0), (65536.0, 1)]
    # consecutive overflows keep halving, and the tracker restarts after each
    assert run([1, 1, 1, 0], 2) == [(32768.0, 0), (16384.0, 0), (8192.0, 0), (8192.0, 1)]


def test_invariants_random_sequences():
    rng = np.random.default_rng(0)
    for interval in (1, 2, 7, 100):
        found = (rng.random(3000) < 0.05).astype(int)
        for s, t in run(found, interval):
            if np.isfinite(s):  # the page's update() has no overflow guard
                m, e = np.frexp(s)
                assert m == 0.5  # stays a power of two
            assert 0 <= t < interval


def f16(vals):
    return np.asarray(vals, np.float32).astype(np.float16).view(np.uint16).copy()


def test_unscale_power_of_two_is_exact():
    # g * 2^-k is exact in fp16 as long as it stays normal: compare with numpy
    rng = np.random.default_rng(1)
    g = f16(rng.normal(0, 1.0, 10000) * 300)
    ref = (g.view(np.float16).astype(np.float32) * np.float32(2.0 ** -4)).astype(np.float16)
    found = O.unscale_check([g], 16.0, 0)
    assert found == 0
    assert np.array_equal(g, ref.view(np.uint16))


def test_unscale_rounds_once_and_reaches_subnormals():
    # values that land in fp16 subnormals: a single RNE rounding of the fp32 product,
    # as numpy's fp32 -> fp16 cast does it
    rng = np.random.default_rng(2)
    g = f16(rng.normal(0, 1e-5, 20000) * 65536.0)
    ref = (g.view(np.float16).astype(np.float32) * np.float32(1.0 / 65536.0)).astype(np.float16)
    assert O.unscale_check([g], 65536.0, 0) == 0
    assert np.array_equal(g, ref.view(np.uint16))
    assert np.any((g & 0x7C00) == 0) and np.any(g & 0x03FF)  # some subnormals present
    # a non-power-of-two scale: the inverse is the fp32 reciprocal
    g = f16(rng.normal(0, 1.0, 5000))
    inv = np.float32(1.0) / np.float32(3.0)
    ref = (g.view(np.float16).astype(np.float32) * inv).astype(np.float16)
    O.unscale_check([g], 3.0, 0)
    assert np.array_equal(g, ref.view(np.uint16))


@pytest.mark.parametrize("bits", [0x7C00, 0xFC00, 0x7E00, 0xFE01])
def test_unscale_detects_injected_nonfinite(bits):
    g1 = f16(np.linspace(-2, 2, 1000))
    g2 = f16(np.linspace(-1, 1, 333))
    g2[100] = bits
    assert O.unscale_check([g1, g2], 1024.0, 0) == 1
    assert O.unscale_check([f16([1.0, 2.0])], 1024.0, 1) == 1  # OR-accumulated
    assert O.unscale_check([f16([1.0, 2.0])], 1024.0, 0) == 0


def test_unscale_overflow_after_scaling_is_flagged():
    # a scale below one can push a finite fp16 past 65504: flagged on the stored value
    g = f16([60000.0, 1.0])
    assert O.unscale_check([g], 0.5, 0) == 1
    assert g[0] == 0x7C00


def test_skip_and_backoff_flow():
    """loss*S -> backward -> unscale -> check -> skip + halve, or step [PT-CH20 §20.2.2]."""
    st = O.ScalerState(np.float32(65536.0), 5)
    g = f16([1.0, 2.0, 3.0])
    g[1] = 0x7C00
    found = O.unscale_check([g], float(st.scale), 0)
    stepped = not found
    st = O.update_scale(st, found, 2.0, 0.5, 2000)
    assert not stepped and float(st.scale) == 32768.0 and st.tracker == 0
