"""fp8_amax_f16 / fp8_quantize_f16: the cast of fp16 tensors (an fp16 model
under loss scaling) against the oracle's fp16-input cast [FP8-TRAIN §2;
PT-CH20 §20.2.2].  Amax, scales, codes and transposed codes bit for bit, on the
tiled, flat and per-element paths, at cached and streaming sizes, with fp16
special values."""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
import workloads as W
from tests.parity import assert_codes_equal
from tests.test_gpu_kernels import check_rec, dev_f16

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
@pytest.mark.parametrize("shape,with_t", [((64, 80), True), ((1000, 777), True), ((1000, 777), False),
                                          ((4096, 4096), True), ((8192, 16384), True),
                                          ((3, 5), False)])
def test_f16_cast_matches_oracle(fmt, shape, with_t):
    sigma = 1.0 if fmt == F.E4M3FN else 1e-4 * 65536.0
    x = W.normal_f16(81, fmt, shape, sigma)
    ref = O.to_fp8(x, fmt, with_transpose=with_t, in_fmt=O.F16)
    xd = dev_f16(x).reshape(shape)
    rec = F.ScaleRec()
    q = torch.empty(shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty((shape[1], shape[0]), dtype=torch.uint8, device=DEV) if with_t else None
    F.fp8_amax_f16(xd, rec)
    F.fp8_quantize_f16(xd, fmt, rec, q, qT)
    torch.cuda.synchronize()
    check_rec(rec, ref.sc, f"{shape}")
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, "codes")
    if with_t:
        assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, "transposed codes")


@pytest.mark.parametrize("special", ["inf", "nan", "subnormals", "max_f16", "zeros"])
def test_f16_cast_special_values(special):
    x = W.normal_f16(82, 1, (128, 96), 2.0)
    if special == "inf":
        x[5, 7] = 0xFC00
    elif special == "nan":
        x[100, 0] = 0x7E01
    elif special == "subnormals":
        x[:] = np.arange(x.size, dtype=np.uint16).reshape(x.shape) % 0x0400  # all fp16 subnormals
    elif special == "max_f16":
        x[0, 0] = 0x7BFF  # 65504
    else:
        x[:] = 0x8000
    for fmt in (F.E4M3FN, F.E5M2):
        ref = O.to_fp8(x, fmt, in_fmt=O.F16)
        xd = dev_f16(x).reshape(x.shape)
        rec = F.ScaleRec()
        q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        qT = torch.empty((x.shape[1], x.shape[0]), dtype=torch.uint8, device=DEV)
        F.fp8_amax_f16(xd, rec)
        F.fp8_quantize_f16(xd, fmt, rec, q, qT)
        torch.cuda.synchronize()
        check_rec(rec, ref.sc, special)
        assert_codes_equal(fmt, q.cpu().numpy(), ref.q, special)
        assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, special)
