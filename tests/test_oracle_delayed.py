"""Pins for the oracle's delayed scaling ["第20章 量化与混合精度训练", §20.5.9:
each FP8 op keeps an amax history of its input and takes every step's scale
from the amax of earlier steps].  The pins use what that description and the
already pinned dynamic path fix: with an unchanging tensor, delayed and
dynamic scaling agree; a history of length 1 is exactly "the previous step's
amax"; a window of H steps forgets older entries (closed form with powers of
two); a tensor that outgrows its history saturates at the format maximum."""
import numpy as np
import pytest

import oracle as O
import workloads as W


def bf16(seed, shape, sigma):
    return W.normal_bf16(seed, 0, shape, sigma)


def pow2_tensor(e, shape=(16, 32)):
    """bf16 tensor whose largest magnitude is exactly 2^e (the rest smaller)."""
    x = W.normal_bf16(3, 0, shape, 2.0 ** e / 8)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    f = np.clip(f, -(2.0 ** e) * 0.9, 2.0 ** e * 0.9).astype(np.float32)
    f.flat[5] = 2.0 ** e
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
def test_steady_tensor_matches_dynamic(fmt):
    x = bf16(11, (48, 64), 1.0)
    hist = np.zeros(4, np.float32)
    hist[0] = O.bits_to_f32(O.amax_bits(x))  # seeded with the tensor's own amax
    dyn = O.to_fp8(x, fmt)
    for _ in range(6):
        d = O.to_fp8_delayed(x, fmt, hist)
        assert np.array_equal(d.q, dyn.q) and np.array_equal(d.qT, dyn.qT)
        assert d.sc == dyn.sc
        hist = d.hist


def test_history_of_one_is_the_previous_step():
    xs = [bf16(20 + t, (32, 32), 10.0 ** (t % 3 - 1)) for t in range(6)]
    hist = np.array([O.bits_to_f32(O.amax_bits(xs[0]))], np.float32)
    for t in range(1, 6):
        d = O.to_fp8_delayed(xs[t], O.E4M3FN, hist)
        prev = O.to_fp8(xs[t - 1], O.E4M3FN)  # dynamic scaling of the previous step's tensor
        assert d.sc == prev.sc
        assert np.array_equal(d.q, O.quantize(xs[t], O.E4M3FN, prev.sc.scale32))
        assert d.amax_bits == O.amax_bits(xs[t])
        hist = d.hist


@pytest.mark.parametrize("H", [1, 3, 8])
def test_window_forgets_older_steps(H):
    # amax halves every step: 2^0, 2^-1, ...; with a window of H the largest
    # remembered amax at step t is 2^-(t-H), so scale = 448 * 2^(t-H) exactly
    hist = np.zeros(H, np.float32)
    hist[0] = 1.0
    for t in range(1, 12):
        x = pow2_tensor(-t)
        d = O.to_fp8_delayed(x, O.E4M3FN, hist)
        oldest = max(t - H, 0)
        assert d.sc.scale == 448.0 * 2.0 ** oldest
        assert d.sc.inv == 2.0 ** -oldest / 448.0
        assert d.amax_bits == np.float32(2.0 ** -t).view(np.uint32)
        assert d.hist[0] == np.float32(2.0 ** -t) and d.hist.size == H
        hist = d.hist


def test_growing_tensor_saturates():
    small, big = pow2_tensor(0), pow2_tensor(3)  # the amax grows 8x in one step
    hist = np.array([1.0], np.float32)
    d = O.to_fp8_delayed(big, O.E4M3FN, hist)
    # scale 448: every |x| > 1 clamps to the largest code 0x7E (448)
    f = (big.astype(np.uint32) << 16).view(np.float32)
    sat = np.abs(f) > 1.0
    assert sat.any()
    assert np.all((d.q[sat] & 0x7F) == 0x7E)
    assert np.array_equal(d.q[~sat], O.quantize(big, O.E4M3FN, np.float32(448.0))[~sat])
    assert O.to_fp8_delayed(small, O.E4M3FN, d.hist).sc.scale == 448.0 / 8.0


def test_nan_in_history_makes_every_code_nan():
    x = bf16(30, (8, 16), 1.0)
    d = O.to_fp8_delayed(x, O.E4M3FN, np.array([1.0, np.nan, 2.0], np.float32))
    assert np.isnan(d.sc.scale)
    assert np.all((d.q & 0x7F) == 0x7F)


def test_push_order():
    h = np.array([4.0, 3.0, 2.0], np.float32)
    d = O.to_fp8_delayed(pow2_tensor(4), O.E5M2, h)
    assert d.hist.tolist() == [16.0, 4.0, 3.0]
    assert d.sc.scale == 57344.0 / 4.0
