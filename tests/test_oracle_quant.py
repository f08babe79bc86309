"""Pins for the oracle's amax, fp64 scale and quantize-cast [FP8-TRAIN §2, §3].

Independent references: torch's CPU ops running the page's own formula
(abs().max(), fp64 division, fp32 multiply, clamp, cast), closed forms for
power-of-two inputs, and invariants.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from conftest import golden

TORCH_FP8 = {O.E4M3FN: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2}


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def torch_chain(x_bits, fmt, eps=1e-12):
    """The page's to_fp8 chain executed by torch on the CPU [FP8-TRAIN §2]."""
    x = bf16_tensor(x_bits)
    fmax = torch.finfo(TORCH_FP8[fmt]).max
    amax = x.float().abs().max()
    # A true fp64 division, as the page intends.  (torch evaluates python_float / tensor
    # as reciprocal-then-multiply, which can land one fp64 ulp away.)
    scale = torch.full((), fmax, dtype=torch.float64) / amax.double().clamp(min=eps)
    q = (x.float() * scale).clamp(-fmax, fmax).to(TORCH_FP8[fmt])
    inv = scale.reciprocal()
    return float(amax), float(scale), float(inv), q.view(torch.uint8).numpy()


def sample_inputs():
    yield "normal", W.normal_bf16(11, 1, (97, 131), 1.0)
    yield "weights", W.normal_bf16(11, 2, (64, 200), 0.02)
    yield "grads", W.normal_bf16(11, 3, (50, 77), 1e-4)
    yield "outliers", W.normal_bf16(11, 4, (128, 96), 1.0, 0.01, 50.0)
    yield "logmag", W.logmag_bf16(11, 5, (4096,), -6.0, 3.0)
    yield "logmag_grad", W.logmag_bf16(11, 6, (4096,), -8.0, -2.0)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
def test_quantize_matches_torch_chain(fmt):
    for name, x in sample_inputs():
        amax, s, inv, q_ref = torch_chain(x, fmt)
        qz = O.to_fp8(x, fmt, with_transpose=False)
        assert O.bits_to_f32(qz.sc.amax_bits) == amax, name
        assert qz.sc.scale == s and qz.sc.inv == inv, name
        assert np.array_equal(qz.q.reshape(-1), q_ref.reshape(-1)), name


def test_amax_invariants():
    x = W.normal_bf16(12, 1, (5000,), 3.0)
    a = O.amax_bits(x)
    # the definition via an independent path: torch decode, numpy max
    ref = np.abs(bf16_tensor(x).float().numpy()).max()
    assert O.bits_to_f32(a) == ref
    # order-free
    perm = np.random.default_rng(0).permutation(x.size)
    assert O.amax_bits(x[perm]) == a
    # sign-free: negating every element (flip bf16 sign bit) keeps amax
    assert O.amax_bits(x ^ np.uint16(0x8000)) == a
    # all zeros (both signs) and empty
    assert O.amax_bits(np.array([0x0000, 0x8000], np.uint16)) == 0
    assert O.amax_bits(np.array([], np.uint16)) == 0
    # NaN propagates, inf is the max
    y = x.copy()
    y[17] = 0x7FC1
    assert np.isnan(O.bits_to_f32(O.amax_bits(y)))
    y[17] = 0xFF80  # -inf
    assert O.bits_to_f32(O.amax_bits(y)) == np.inf


def test_scale_closed_forms_and_power_of_two_invariance():
    def f32_bits(v):
        return int(np.array([v], np.float32).view(np.uint32)[0])

    # amax 1.75 (e4m3): 448/1.75 = 256, inverse 2^-8, both exact
    sc = O.scale_from_amax(f32_bits(1.75), O.E4M3FN)
    assert sc.scale == 256.0 and sc.inv == 2.0 ** -8
    sc = O.scale_from_amax(f32_bits(57344.0), O.E5M2)
    assert sc.scale == 1.0 and sc.inv == 1.0
    # power-of-two invariance: amax * 2^k -> scale / 2^k and inverse * 2^k exactly
    base = O.scale_from_amax(f32_bits(3.1), O.E4M3FN)
    for k in (-20, -3, 5, 30):
        sk = O.scale_from_amax(f32_bits(np.float32(3.1) * np.float32(2.0 ** k)), O.E4M3FN)
        assert sk.scale == base.scale / 2.0 ** k
        assert sk.inv == base.inv * 2.0 ** k
    # scale is fp64 division of the fp32 amax; inverse is the fp64 reciprocal of the scale
    a = np.float32(0.3)
    sc = O.scale_from_amax(f32_bits(a), O.E4M3FN)
    assert sc.scale == 448.0 / float(a) and sc.inv == 1.0 / (448.0 / float(a))
    assert sc.scale32 == np.float32(sc.scale) and sc.inv32 == np.float32(sc.inv)
    # zero amax -> clamped to EPS; inf amax -> scale 0
    sc = O.scale_from_amax(0, O.E4M3FN)
    assert sc.scale == 448.0 / 1e-12
    sc = O.scale_from_amax(f32_bits(np.inf), O.E4M3FN)
    assert sc.scale == 0.0 and sc.inv == np.inf
    sc = O.scale_from_amax(0x7FC00000, O.E5M2)
    assert np.isnan(sc.scale) and np.isnan(sc.inv)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
def test_quantize_invariants(fmt):
    x = W.normal_bf16(13, 1, (64, 48), 0.7)
    qz = O.to_fp8(x, fmt)
    # the max-magnitude element encodes to the largest finite code
    mc = O.max_code(fmt)
    i = np.argmax(np.abs(bf16_tensor(x).float().numpy()))
    assert (int(qz.q.reshape(-1)[i]) & 0x7F) == mc
    # no code past the largest finite one
    assert np.all((qz.q & 0x7F) <= mc)
    # power-of-two scaling of the input leaves the codes unchanged
    x2 = bf16_tensor(x).float().numpy() * 8.0
    x2 = W.f32_to_bf16_bits(x2).reshape(x.shape)
    q2 = O.to_fp8(x2, fmt)
    assert np.array_equal(q2.q, qz.q) and q2.sc.inv == qz.sc.inv * 8.0
    # transposed copy
    assert np.array_equal(qz.qT, qz.q.T)
    assert np.array_equal(O.transpose(qz.qT), qz.q)


def test_quantize_special_inputs():
    # +-inf saturate to the max code under a finite scale; NaN stays NaN; -0 keeps its sign
    x = np.array([0x3F80, 0x7F80, 0xFF80, 0x7FC0, 0x8000, 0x0000], np.uint16)  # 1, inf, -inf, nan, -0, 0
    q = O.quantize(x, O.E4M3FN, np.float32(2.0))
    assert q[0] == O.encode(O.E4M3FN, [2.0])[0]
    assert q[1] == 0x7E and q[2] == 0xFE
    assert np.isnan(O.decode(O.E4M3FN, q[3:4])[0])
    assert q[4] == 0x80 and q[5] == 0x00
    # scale 0 (amax inf): finite -> +-0, inf -> NaN
    q = O.quantize(x, O.E5M2, np.float32(0.0))
    assert q[0] == 0x00 and np.isnan(O.decode(O.E5M2, q[1:2])[0])


def test_scale_direction_trap():
    """Passing the inverse scales recovers x @ W^T; passing the scales is off by
    (s_x * s_w)^2 [FP8-TRAIN §2]."""
    assert golden("scale_direction.json")["wrong_direction_factor"] == "(s_a * s_b)^2"
    x = W.normal_bf16(14, 1, (32, 64), 1.0)
    w = W.normal_bf16(14, 2, (48, 64), 0.02)
    xf = bf16_tensor(x).double().numpy()
    wf = bf16_tensor(w).double().numpy()
    exact = xf @ wf.T
    fw = O.linear_fwd(x, w)
    err = np.abs(fw.c - exact).max() / np.abs(exact).max()
    assert err < 0.08  # FP8 e4m3 quantisation error of both operands
    wrong = O.gemm(fw.x.q, O.E4M3FN, fw.w.q, O.E4M3FN, fw.x.sc.scale, fw.w.sc.scale)
    ratio = np.median(np.abs(wrong) / np.maximum(np.abs(fw.c), 1e-30))
    factor = (fw.x.sc.scale * fw.w.sc.scale) ** 2
    assert abs(ratio / factor - 1) < 1e-5


# ----------------------------------------------- fp16 inputs (an fp16 model)

def f16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.float16)


def torch_chain_f16(x_bits, fmt, eps=1e-12):
    """The page's to_fp8 chain on an fp16 tensor, executed by torch on the CPU."""
    x = f16_tensor(x_bits)
    fmax = torch.finfo(TORCH_FP8[fmt]).max
    amax = x.float().abs().max()
    scale = torch.full((), fmax, dtype=torch.float64) / amax.double().clamp(min=eps)
    q = (x.float() * scale).clamp(-fmax, fmax).to(TORCH_FP8[fmt])
    return float(amax), float(scale), float(scale.reciprocal()), q.view(torch.uint8).numpy()


def f16_inputs():
    yield "normal", W.normal_f16(13, 1, (97, 131), 1.0)
    yield "grads_scaled", W.normal_f16(13, 2, (64, 200), 1e-4 * 65536.0)
    yield "small", W.normal_f16(13, 3, (50, 77), 1e-5)  # fp16 subnormals among them
    yield "wide", W.normal_f16(13, 4, (4096,), 2000.0)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
def test_f16_input_quantize_matches_torch_chain(fmt):
    for name, x in f16_inputs():
        amax, s, inv, q_ref = torch_chain_f16(x, fmt)
        qz = O.to_fp8(x, fmt, with_transpose=False, in_fmt=O.F16)
        assert O.bits_to_f32(qz.sc.amax_bits) == amax, name
        assert qz.sc.scale == s and qz.sc.inv == inv, name
        assert np.array_equal(qz.q.reshape(-1), q_ref.reshape(-1)), name


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
def test_f16_and_bf16_inputs_of_the_same_values_cast_alike(fmt):
    """Values representable in both formats (8 significant bits or fewer, in the
    common exponent range) give the same amax, scale and codes whichever
    format carries them: a wrong fp16 decode breaks this."""
    rng = np.random.default_rng(14)
    mant = rng.integers(128, 256, 3000).astype(np.float64)   # 8 significant bits
    expo = rng.integers(-14, 8, 3000).astype(np.float64)  # fp16 normal range
    sign = rng.choice([-1.0, 1.0], 3000)
    v = (sign * mant * 2.0 ** (expo - 7)).astype(np.float32)
    f16 = v.astype(np.float16)
    assert np.array_equal(f16.astype(np.float32), v)        # exact in fp16
    b16 = W.f32_to_bf16_bits(v)
    assert np.array_equal((b16.astype(np.uint32) << 16).view(np.float32), v)  # exact in bf16
    a = O.to_fp8(f16.view(np.uint16), fmt, with_transpose=False, in_fmt=O.F16)
    b = O.to_fp8(b16, fmt, with_transpose=False)
    assert a.sc.amax_bits == b.sc.amax_bits and a.sc.scale == b.sc.scale
    assert np.array_equal(a.q, b.q)


def test_f16_amax_special_values():
    x = W.normal_f16(15, 1, (1000,), 3.0)
    ref = np.abs(x.view(np.float16).astype(np.float32)).max()
    assert O.bits_to_f32(O.amax_bits(x, O.F16)) == ref
    y = x.copy()
    y[5] = 0xFC00  # -inf
    assert O.bits_to_f32(O.amax_bits(y, O.F16)) == np.inf
    y[7] = 0x7E01  # NaN
    assert O.amax_bits(y, O.F16) == 0x7FC00000
    assert O.amax_bits(np.array([0x8000, 0x0000, 0x0001], np.uint16), O.F16) == \
        int(np.float32(2.0 ** -24).view(np.uint32))  # smallest fp16 subnormal
