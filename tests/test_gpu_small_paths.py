"""The small-problem paths of the linear entry points, on both sides of their
thresholds: tensors of at most 64 Ki elements are cast by one block that also
reduces their amax, and a backward whose two GEMMs both take the 128 x 128
kernel runs them in one launch.  Codes, transposed codes and scale records
bit-exact against the oracle; every GEMM output within the bound of
tests/parity.py."""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
import workloads as W
from tests.parity import assert_codes_equal, check_gemm_values

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_rec(rec, sc, what):
    r = rec.read()
    assert r["amax_bits"] == sc.amax_bits, what
    assert r["scale"] == sc.scale and r["inv"] == sc.inv, what
    assert 1 <= r["nparts"] <= F.AMAX_PARTS, what


def full_check(got, ref_c, A, fa, B, ia, ib, Kc, ofmt, what):
    R, C = ref_c.shape
    ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(R), np.arange(C), indexing="ij")]
    ad = O.gemm_absdot_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
    check_gemm_values(O.decode(ofmt, host_u16(got)).reshape(-1), ref_c.reshape(-1), ad, Kc, ofmt, what)


# (M, N, K): x = M*K, W = N*K, gy = M*N elements around the 65,536 threshold;
# the last shape puts the backward GEMMs on different kernels (no shared launch)
SHAPES = [(64, 256, 128), (256, 256, 256), (272, 256, 256), (16, 4096, 16), (128, 1040, 64),
          (8192, 256, 1024)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fused", [False, True])
def test_small_layer_paths_match_oracle(shape, fused):
    M, N, K = shape
    x_h = W.normal_bf16(95, 0, (M, K), 1.0, 0.001, 50.0)
    w_h = W.normal_bf16(95, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(95, 2, (M, N), 1e-3 * 65536.0)
    saved = F.LinearSaved(M, N, K)
    ws = F.LinearBwdWs(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
    scale = torch.tensor([65536.0], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.fp8_scaled_linear_fwd(dev_bf16(x_h), dev_bf16(w_h), saved, y)
    if fused:
        F.fp8_scaled_linear_bwd_unscale(dev_bf16(gy_h), saved, ws, scale, found, gx, gw)
    else:
        F.fp8_scaled_linear_bwd(dev_bf16(gy_h), saved, ws, gx, gw, F.OUT_F16)
    torch.cuda.synchronize()
    fw = O.linear_fwd(x_h, w_h)
    bw = O.linear_bwd(gy_h, fw, O.F16)
    for rec, sc, nm in ((saved.x_sc, fw.x.sc, "x"), (saved.w_sc, fw.w.sc, "W"), (ws.gy_sc, bw.gy.sc, "gy")):
        check_rec(rec, sc, nm)
    for got, ref, fmt, nm in ((saved.x_q, fw.x.q, O.E4M3FN, "x_q"), (saved.x_qT, fw.x.qT, O.E4M3FN, "x_qT"),
                              (saved.w_q, fw.w.q, O.E4M3FN, "w_q"), (saved.w_qT, fw.w.qT, O.E4M3FN, "w_qT"),
                              (ws.gy_q, bw.gy.q, O.E5M2, "gy_q"), (ws.gy_qT, bw.gy.qT, O.E5M2, "gy_qT")):
        assert_codes_equal(fmt, got.cpu().numpy(), ref, nm)
    full_check(y, fw.c, fw.x.q, O.E4M3FN, fw.w.q, fw.x.sc.inv, fw.w.sc.inv, K, O.BF16, "y")
    post = float(np.float32(1.0) / np.float32(65536.0)) if fused else 1.0
    full_check(gx, bw.c_gx.astype(np.float64) * post, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.sc.inv * post,
               fw.w.sc.inv, N, O.F16, "gx")
    full_check(gw, bw.c_gw.astype(np.float64) * post, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.sc.inv * post,
               fw.x.sc.inv, M, O.F16, "gw")
    assert int(found.item()) == 0
