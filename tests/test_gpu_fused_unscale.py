"""GPU parity of fp8_scaled_linear_bwd_unscale: the backward GEMMs with the
GradScaler's unscale and non-finite check ["第20章 量化与混合精度训练",
§20.2.2] fused into their fp16 epilogues.

  - bit-identical outputs and flag to the unfused pair fp8_scaled_linear_bwd
    (fp16) + amp_unscale_check over gx and gW (same kernels, same order);
  - against the oracle: codes and scales bit-exact, and every unscaled output
    within the GEMM bound of tests/parity.py scaled by 1/scale (plus one fp16
    unit for the two roundings);
  - the flag: set by an overflow before or after the unscale, never cleared.
"""
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


def run_both(x_h, w_h, gy_h, scale_val, found0=0):
    """The fused entry point and the unfused pair on the same forward state."""
    M, K = x_h.shape
    N = w_h.shape[0]
    saved = F.LinearSaved(M, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_scaled_linear_fwd(dev_bf16(x_h), dev_bf16(w_h), saved, y)
    gy = dev_bf16(gy_h)
    scale = torch.tensor([scale_val], dtype=torch.float32, device=DEV)
    outs = {}
    for fused in (True, False):
        ws = F.LinearBwdWs(M, N)
        gx = torch.full((M, K), 7.0, dtype=torch.float16, device=DEV)
        gw = torch.full((N, K), 7.0, dtype=torch.float16, device=DEV)
        found = torch.full((1,), found0, dtype=torch.int32, device=DEV)
        if fused:
            F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        else:
            F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, F.OUT_F16)
            F.amp_unscale_check([gx, gw], scale, found)
        torch.cuda.synchronize()
        outs[fused] = (host_u16(gx), host_u16(gw), int(found.item()), ws)
    return saved, outs


SHAPES = [(64, 256, 128),      # the small layer: 128 x 128 kernel
          (272, 144, 400),     # ragged tiles, K not a multiple of 128
          (2048, 4096, 2048),  # 256 x 256 kernel for both GEMMs
          (2064, 4000, 1040)]  # 256 x 256 kernel with ragged M, N and K


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scale", [65536.0, 49152.0, 1000.0])
def test_fused_unscale_is_the_unfused_pair_bit_for_bit(shape, scale):
    """Both roundings of each element (fp16 of acc * alpha, then fp16 of its
    product with fl32(1/scale), inexact unless the scale is a power of two)
    must be those of the unfused pair."""
    M, N, K = shape
    x_h = W.normal_bf16(81, 0, (M, K), 1.0, 0.001, 50.0)
    w_h = W.normal_bf16(81, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(81, 2, (M, N), 1e-4 * scale)
    _, outs = run_both(x_h, w_h, gy_h, scale)
    for i, what in ((0, "gx"), (1, "gw")):
        assert np.array_equal(outs[True][i], outs[False][i]), what
    assert outs[True][2] == outs[False][2] == 0


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_fused_unscale_matches_oracle(shape):
    M, N, K = shape
    x_h = W.normal_bf16(82, 0, (M, K), 1.0)
    w_h = W.normal_bf16(82, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(82, 2, (M, N), 1e-4 * 65536.0)
    scale = 65536.0
    _, outs = run_both(x_h, w_h, gy_h, scale)
    gx, gw, found, ws = outs[True]
    fw = O.linear_fwd(x_h, w_h)
    bw = O.linear_bwd(gy_h, fw, O.F16)
    assert_codes_equal(O.E5M2, ws.gy_q.cpu().numpy(), bw.gy.q, "gy_q")
    assert_codes_equal(O.E5M2, ws.gy_qT.cpu().numpy(), bw.gy.qT, "gy_qT")
    inv_s = float(np.float32(1.0) / np.float32(scale))
    rng = np.random.default_rng(M + N + K)
    for got, c_ref, A, B, ia, ib, Kc, what in (
            (gx, bw.c_gx, bw.gy.q, fw.w.qT, bw.gy.sc.inv, fw.w.sc.inv, N, "gx"),
            (gw, bw.c_gw, bw.gy.qT, fw.x.qT, bw.gy.sc.inv, fw.x.sc.inv, M, "gw")):
        R, C = c_ref.shape
        if R * C <= 1 << 20:
            ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(R), np.arange(C), indexing="ij")]
        else:
            ii, jj = rng.integers(0, R, 4000), rng.integers(0, C, 4000)
        absdot = O.gemm_absdot_at(A, O.E5M2, B, O.E4M3FN, ia, ib, ii, jj)
        g = O.decode(O.F16, got.reshape(R, C)[ii, jj])
        check_gemm_values(g, c_ref[ii, jj].astype(np.float64) * inv_s, absdot * inv_s, Kc, O.F16,
                          what)
    assert found == 0


def test_fused_unscale_flags_overflow():
    """A loss scale of 2^-12 makes the unscaled gradients overflow fp16; a
    huge gradient entry makes the scaled product itself overflow.  Both set
    the flag exactly as the unfused pass does, inf positions included."""
    M, N, K = 256, 512, 384
    x_h = W.normal_bf16(83, 0, (M, K), 1.0)
    w_h = W.normal_bf16(83, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(83, 2, (M, N), 1e-4 * 65536.0)
    _, outs = run_both(x_h, w_h, gy_h, 2.0 ** -12)
    assert outs[True][2] == outs[False][2] == 1
    for i in (0, 1):
        assert np.array_equal(outs[True][i], outs[False][i])
    # |gW| ~ 100 before the unscale: x 4096 overflows; |gx| ~ 3 stays finite
    assert np.any((outs[True][1] & 0x7FFF) == 0x7C00)
    assert not np.any((outs[True][0] & 0x7FFF) >= 0x7C00)
    big = gy_h.copy()
    big[3, 5] = W.f32_to_bf16_bits(np.array([3.0e9], np.float32))[0]
    _, outs = run_both(x_h, w_h, big, 65536.0)
    assert outs[True][2] == outs[False][2] == 1
    for i in (0, 1):
        assert np.array_equal(outs[True][i], outs[False][i])


def test_fused_unscale_never_clears_the_flag():
    M, N, K = 128, 256, 128
    x_h = W.normal_bf16(84, 0, (M, K), 1.0)
    w_h = W.normal_bf16(84, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(84, 2, (M, N), 1e-4 * 65536.0)
    _, outs = run_both(x_h, w_h, gy_h, 65536.0, found0=1)
    assert outs[True][2] == outs[False][2] == 1


@pytest.mark.parametrize("fa,fb", [(F.E4M3FN, F.E4M3FN), (F.E5M2, F.E4M3FN), (F.E4M3FN, F.E5M2),
                                   (F.E5M2, F.E5M2)])
@pytest.mark.parametrize("shape", [(144, 272, 400), (2064, 4000, 1040), (912, 13072, 400)])
def test_gemm_unscale_is_gemm_then_unscale(fa, fb, shape):
    """fp8_gemm_unscale = fp8_gemm (fp16 out) followed by amp_unscale_check on
    its output, bit for bit, flag included."""
    M, N, K = shape
    rng = np.random.default_rng(M + 7 * N + K + 10 * fa + fb)
    A = rng.integers(0, 256, (M, K), dtype=np.int64).astype(np.uint8)
    B = rng.integers(0, 256, (N, K), dtype=np.int64).astype(np.uint8)
    A[~np.isfinite(O.decode(fa, A))] = 0
    B[~np.isfinite(O.decode(fb, B))] = 0
    Ad, Bd = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    inv = torch.tensor([2.0 ** -9 / 3.0, 0.37 / 448.0 * 2.0 ** -14], dtype=torch.float64,
                       device=DEV)
    scale = torch.tensor([49152.0], dtype=torch.float32, device=DEV)
    C1 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    C2 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    f1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    f2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.fp8_gemm_unscale(Ad, fa, Bd, fb, inv.data_ptr(), inv.data_ptr() + 8, scale, f1, C1)
    F.fp8_gemm(Ad, fa, Bd, fb, inv.data_ptr(), inv.data_ptr() + 8, C2, F.OUT_F16)
    F.amp_unscale_check([C2], scale, f2)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(C1), host_u16(C2))
    assert int(f1.item()) == int(f2.item())


def run_both_delayed(x_h, w_h, gy_h, scale_val, hist_len=4):
    """Delayed scaling: the fused backward and the unfused pair from the same
    forward state and the same gy history."""
    M, K = x_h.shape
    N = w_h.shape[0]
    x, w, gy = dev_bf16(x_h), dev_bf16(w_h), dev_bf16(gy_h)
    saved = F.LinearSaved(M, N, K)
    hx = torch.full((hist_len,), 3.0, dtype=torch.float32, device=DEV)
    hw = torch.full((hist_len,), 0.05, dtype=torch.float32, device=DEV)
    F.fp8_scaled_linear_fwd_delayed(x, w, saved, hx, hw, torch.empty((M, N), dtype=torch.bfloat16,
                                                                      device=DEV))
    # gy's history: its own amax (the delayed scale then equals the dynamic one)
    gy_amax = float(np.abs(O.decode(O.BF16, gy_h).astype(np.float64)).max())
    hg0 = torch.full((hist_len,), gy_amax, dtype=torch.float32, device=DEV)
    scale = torch.tensor([scale_val], dtype=torch.float32, device=DEV)
    outs = {}
    for fused in (True, False):
        ws = F.LinearBwdWs(M, N)
        hg = hg0.clone()
        gx = torch.full((M, K), 7.0, dtype=torch.float16, device=DEV)
        gw = torch.full((N, K), 7.0, dtype=torch.float16, device=DEV)
        found = torch.zeros(1, dtype=torch.int32, device=DEV)
        if fused:
            F.fp8_scaled_linear_bwd_delayed_unscale(gy, saved, ws, hg, scale, found, gx, gw)
        else:
            F.fp8_scaled_linear_bwd_delayed(gy, saved, ws, hg, gx, gw, F.OUT_F16)
            F.amp_unscale_check([gx, gw], scale, found)
        torch.cuda.synchronize()
        outs[fused] = (host_u16(gx), host_u16(gw), int(found.item()), hg.cpu().numpy(),
                       ws.gy_q.cpu().numpy(), ws.gy_qT.cpu().numpy())
    return outs


def run_both_rowwise(x_h, w_h, gy_h, scale_val):
    M, K = x_h.shape
    N = w_h.shape[0]
    x, w, gy = dev_bf16(x_h), dev_bf16(w_h), dev_bf16(gy_h)
    saved = F.LinearSavedRW(M, N, K)
    F.fp8_scaled_linear_fwd_rowwise(x, w, saved, torch.empty((M, N), dtype=torch.bfloat16,
                                                             device=DEV))
    scale = torch.tensor([scale_val], dtype=torch.float32, device=DEV)
    outs = {}
    for fused in (True, False):
        ws = F.LinearBwdWsRW(M, N)
        gx = torch.full((M, K), 7.0, dtype=torch.float16, device=DEV)
        gw = torch.full((N, K), 7.0, dtype=torch.float16, device=DEV)
        found = torch.zeros(1, dtype=torch.int32, device=DEV)
        if fused:
            F.fp8_scaled_linear_bwd_rowwise_unscale(gy, saved, ws, scale, found, gx, gw)
        else:
            F.fp8_scaled_linear_bwd_rowwise(gy, saved, ws, gx, gw, F.OUT_F16)
            F.amp_unscale_check([gx, gw], scale, found)
        torch.cuda.synchronize()
        outs[fused] = (host_u16(gx), host_u16(gw), int(found.item()),
                       ws.gy_row_inv.cpu().numpy(), ws.gy_q.cpu().numpy(), ws.gy_qT.cpu().numpy())
    return outs


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scale", [65536.0, 1000.0])
@pytest.mark.parametrize("mode", ["delayed", "rowwise"])
def test_delayed_and_rowwise_fused_unscale_are_the_unfused_pair(mode, shape, scale):
    """Delayed and row-wise scaling: the fused backward stores the unfused
    pair's bits (gradients, flag, gy codes and gy's history or scale vector)."""
    M, N, K = shape
    x_h = W.normal_bf16(85, 0, (M, K), 1.0, 0.001, 50.0)
    w_h = W.normal_bf16(85, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(85, 2, (M, N), 1e-4 * scale)
    outs = (run_both_delayed if mode == "delayed" else run_both_rowwise)(x_h, w_h, gy_h, scale)
    for i, what in enumerate(("gx", "gw", "found", "gy state", "gy_q", "gy_qT")):
        a, b = outs[True][i], outs[False][i]
        assert np.array_equal(a, b) if isinstance(a, np.ndarray) else a == b, what
    assert outs[True][2] == 0


@pytest.mark.parametrize("mode", ["delayed", "rowwise"])
def test_delayed_and_rowwise_fused_unscale_flag_overflow(mode):
    M, N, K = 256, 512, 384
    x_h = W.normal_bf16(86, 0, (M, K), 1.0)
    w_h = W.normal_bf16(86, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(86, 2, (M, N), 1e-4 * 65536.0)
    outs = (run_both_delayed if mode == "delayed" else run_both_rowwise)(x_h, w_h, gy_h, 2.0 ** -12)
    assert outs[True][2] == outs[False][2] == 1
    for i in (0, 1):
        assert np.array_equal(outs[True][i], outs[False][i])
    assert np.any((outs[True][1] & 0x7FFF) == 0x7C00)
