"""Pins the gfx950 FP8 matrix-instruction arithmetic that the GEMM tolerance
(tests/parity.py) is derived from, through fp8_gemm with alpha = 1:
  - every product of two finite FP8 codes (all four format pairings,
    subnormals included) comes out exact;
  - inside one group of 8 consecutive k, a product 2^-13 below the group's
    largest is kept and one 2^-14 below is dropped;
  - the same small product in another group (or another k-tile) is kept down
    to the fp32 limit (2^-23 below), i.e. groups are accumulated in fp32.
"""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gemm_f32(A, fa, B, fb):
    one = torch.ones(2, dtype=torch.float64, device=DEV)
    M, K = A.shape
    C = torch.empty((M, B.shape[0]), dtype=torch.float32, device=DEV)
    F.fp8_gemm(torch.from_numpy(A).to(DEV), fa, torch.from_numpy(B).to(DEV), fb, one.data_ptr(),
               one.data_ptr() + 8, C, F.OUT_F32)
    torch.cuda.synchronize()
    return C.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fa,fb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_every_single_product_is_exact(fa, fb):
    ca = np.arange(256)
    ca[~np.isfinite(O.decode(fa, ca))] = 0
    cb = np.arange(256)
    cb[~np.isfinite(O.decode(fb, cb))] = 0
    A = np.zeros((256, 16), np.uint8)
    B = np.zeros((256, 16), np.uint8)
    A[:, 0] = ca
    B[:, 0] = cb
    C = gemm_f32(A, fa, B, fb)
    assert np.array_equal(C, np.outer(O.decode(fa, ca), O.decode(fb, cb)))


def enc(v):
    return int(O.encode(O.E4M3FN, np.array([v]))[0])


def pow2_pair(e):
    a = max(-6, min(8, e // 2))
    return 2.0 ** a, 2.0 ** (e - a)


def residual(gap, pos, K=128):
    """2^16 at k=0 plus 2^(16-gap) at k=pos: what the device adds on top of 2^16,
    in units of the small term."""
    A = np.zeros((16, K), np.uint8)
    B = np.zeros((16, K), np.uint8)
    for k, e in ((0, 16), (pos, 16 - gap)):
        a, b = pow2_pair(e)
        A[0, k], B[0, k] = enc(a), enc(b)
    return (gemm_f32(A, 0, B, 0)[0, 0] - 2.0 ** 16) / 2.0 ** (16 - gap)


def test_group_alignment_window():
    for pos in (1, 7):  # same group of 8 as k = 0
        assert residual(13, pos) == 1.0
        assert residual(14, pos) == 0.0
    for pos, K in ((8, 128), (64, 128), (127, 128), (200, 256)):  # other groups / k-tiles
        assert residual(23, pos, K) == 1.0
