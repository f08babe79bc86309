"""Every output of the GEMMs the benchmark times, against the oracle, on the
workloads' own operands; the epilogue factor's rounding; empty contractions at
the 256 x 256 kernel's sizes.

The square layer (4096^3: forward, dgrad, wgrad) and the MLP block's down
projection (8192 x 4096 x 14336) run on the 256 x 256 LDS-DMA kernel; the down
projection's weight gradient (4096 x 14336 x 8192) on its 224-row form with the
operands' roles swapped.  Their
codes come from the library's own casts (checked bit for bit against the
oracle's), their fp32 outputs are compared element by element with the
oracle's sequential fp32 GEMM: the elementwise bound of tests/parity.py, the
required 1e-3 relative error against each dot product's magnitude, and the
normwise max|C_gpu - C_ref| / max|C_ref| <= 1e-3 [FP8-TRAIN §2, §4; the
accumulator-precision section of AMP-MP].  The bf16 outputs of the layer
entry points are checked over every element too, one bf16 ulp on top.
"""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
from tests.parity import assert_codes_equal, check_gemm_values
from tests.test_gpu_kernels import dev_bf16, dev_u8, host_u16, check_rec

pytestmark = pytest.mark.gpu
DEV = "cuda"


def every(M, N):
    ii, jj = np.meshgrid(np.arange(M, dtype=np.int64), np.arange(N, dtype=np.int64), indexing="ij")
    return ii.reshape(-1), jj.reshape(-1)


def gemm_f32(A, fa, B, fb, inv_a_ptr, inv_b_ptr):
    C = torch.empty((A.shape[0], B.shape[0]), dtype=torch.float32, device=DEV)
    F.fp8_gemm(A, fa, B, fb, inv_a_ptr, inv_b_ptr, C, F.OUT_F32)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_full(got_f32, got_bf16, A, fa, B, fb, inv_a, inv_b, what):
    """got_f32: the fp32-output GEMM; got_bf16: the layer's bf16 output bits
    (or None).  Both against the oracle's full GEMM, every element."""
    M, K = A.shape
    N = B.shape[0]
    c_ref = O.gemm(A, fa, B, fb, inv_a, inv_b)
    ii, jj = every(M, N)
    absdot = O.gemm_absdot_at(A, fa, B, fb, inv_a, inv_b, ii, jj)
    nw = check_gemm_values(got_f32.reshape(-1), c_ref.reshape(-1), absdot, K, None, what + " fp32")
    assert nw <= 1e-3
    if got_bf16 is not None:
        check_gemm_values(O.decode(O.BF16, got_bf16).reshape(-1), c_ref.reshape(-1), absdot, K,
                          O.BF16, what + " bf16")
    return nw


def test_square_layer_every_output():
    """The square workload (x with 0.1% outliers x50): the layer's casts bit for
    bit, then forward, dgrad and wgrad over all 16.8 M outputs each."""
    from workloads.configs import SQUARE as S
    M, N, K = S.M, S.N, S.K
    x_h, w_h, gy_h = S.x(), S.w(), S.gy()
    saved = F.LinearSaved(M, N, K)
    ws = F.LinearBwdWs(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_scaled_linear_fwd(dev_bf16(x_h).reshape(M, K), dev_bf16(w_h).reshape(N, K), saved, y,
                            F.OUT_BF16)
    F.fp8_scaled_linear_bwd(dev_bf16(gy_h).reshape(M, N), saved, ws, gx, gw, F.OUT_BF16)
    torch.cuda.synchronize()
    xq, wq, gq = O.to_fp8(x_h, O.E4M3FN), O.to_fp8(w_h, O.E4M3FN), O.to_fp8(gy_h, O.E5M2)
    for got, ref, fmt, what in ((saved.x_q, xq.q, O.E4M3FN, "x_q"), (saved.x_qT, xq.qT, O.E4M3FN, "x_qT"),
                                (saved.w_q, wq.q, O.E4M3FN, "w_q"), (saved.w_qT, wq.qT, O.E4M3FN, "w_qT"),
                                (ws.gy_q, gq.q, O.E5M2, "gy_q"), (ws.gy_qT, gq.qT, O.E5M2, "gy_qT")):
        assert_codes_equal(fmt, got.cpu().numpy(), ref, what)
    check_rec(saved.x_sc, xq.sc, "x")
    check_rec(saved.w_sc, wq.sc, "w")
    check_rec(ws.gy_sc, gq.sc, "gy")
    inv = lambda rec: rec.inv_ptr()
    # forward y = x W^T: A = x_q [M,K], B = W_q [N,K]
    c = gemm_f32(saved.x_q, F.E4M3FN, saved.w_q, F.E4M3FN, inv(saved.x_sc), inv(saved.w_sc))
    check_full(c, host_u16(y), xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, "fwd")
    # dgrad gx = gy W: A = gy_q [M,N], B = W_qT [K,N]
    c = gemm_f32(ws.gy_q, F.E5M2, saved.w_qT, F.E4M3FN, inv(ws.gy_sc), inv(saved.w_sc))
    check_full(c, host_u16(gx), gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv, "dgrad")
    # wgrad gW = gy^T x: A = gy_qT [N,M], B = x_qT [K,M]
    c = gemm_f32(ws.gy_qT, F.E5M2, saved.x_qT, F.E4M3FN, inv(ws.gy_sc), inv(saved.x_sc))
    check_full(c, host_u16(gw), gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.sc.inv, xq.sc.inv, "wgrad")


def test_mlp_down_projection_every_output():
    """The MLP block's down projection forward, M=8192, N=4096, Kc=14336 (112
    k-tiles, 512 tiles of 256 x 256): every one of its 33.5 M outputs."""
    from workloads.configs import mlp_linear
    L = mlp_linear("down")
    M, N, K = L.M, L.N, L.K
    x_h, w_h = L.x(), L.w()
    saved = F.LinearSaved(M, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_scaled_linear_fwd(dev_bf16(x_h).reshape(M, K), dev_bf16(w_h).reshape(N, K), saved, y,
                            F.OUT_BF16)
    torch.cuda.synchronize()
    xq, wq = O.to_fp8(x_h, O.E4M3FN, with_transpose=False), O.to_fp8(w_h, O.E4M3FN, with_transpose=False)
    assert_codes_equal(O.E4M3FN, saved.x_q.cpu().numpy(), xq.q, "h codes")
    assert_codes_equal(O.E4M3FN, saved.w_q.cpu().numpy(), wq.q, "W_down codes")
    check_rec(saved.x_sc, xq.sc, "h")
    check_rec(saved.w_sc, wq.sc, "W_down")
    c = gemm_f32(saved.x_q, F.E4M3FN, saved.w_q, F.E4M3FN, saved.x_sc.inv_ptr(), saved.w_sc.inv_ptr())
    check_full(c, host_u16(y), xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, "down fwd")


def test_mlp_down_wgrad_every_output():
    """The MLP block's down-projection weight gradient, gW = gy^T h: M=4096,
    N=14336, Kc=8192.  The launcher runs it with the operands' roles swapped
    (1024 tiles of 224 along N, each written transposed); the codes come from
    the library's casts of gy and h (checked against the oracle's), and all
    58.7 M fp32 outputs are compared with the oracle's; the fused-unscale fp16
    output, as the backward writes it, against the same reference."""
    from workloads.configs import mlp_linear
    from tests.parity import check_unscaled_values
    from bench import loss_scaled, LOSS_SCALE
    L = mlp_linear("down")
    T, H, Fd = L.M, L.N, L.K  # h [T, Fd], W [H, Fd], gy [T, H]
    h_h, gy_h = L.x(), loss_scaled(np, L.gy())
    rec_h, rec_g = F.ScaleRec(), F.ScaleRec()
    h_q = torch.empty((T, Fd), dtype=torch.uint8, device=DEV)
    h_qT = torch.empty((Fd, T), dtype=torch.uint8, device=DEV)
    g_q = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    g_qT = torch.empty((H, T), dtype=torch.uint8, device=DEV)
    hd, gd = dev_bf16(h_h).reshape(T, Fd), dev_bf16(gy_h).reshape(T, H)
    F.fp8_amax(hd, rec_h)
    F.fp8_quantize(hd, F.E4M3FN, rec_h, h_q, h_qT)
    F.fp8_amax(gd, rec_g)
    F.fp8_quantize(gd, F.E5M2, rec_g, g_q, g_qT)
    torch.cuda.synchronize()
    hq, gq = O.to_fp8(h_h, O.E4M3FN), O.to_fp8(gy_h, O.E5M2)
    assert_codes_equal(O.E4M3FN, h_qT.cpu().numpy(), hq.qT, "h^T codes")
    assert_codes_equal(O.E5M2, g_qT.cpu().numpy(), gq.qT, "gy^T codes")
    check_rec(rec_h, hq.sc, "h")
    check_rec(rec_g, gq.sc, "gy")
    del h_q, g_q
    # gW = gy^T h: A = gy_qT [H, T], B = h_qT [Fd, T]
    c = gemm_f32(g_qT, F.E5M2, h_qT, F.E4M3FN, rec_g.inv_ptr(), rec_h.inv_ptr())
    scale = torch.tensor([LOSS_SCALE], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    gw = torch.empty((H, Fd), dtype=torch.float16, device=DEV)
    F.fp8_gemm_unscale(g_qT, F.E5M2, h_qT, F.E4M3FN, rec_g.inv_ptr(), rec_h.inv_ptr(), scale, found, gw)
    torch.cuda.synchronize()
    assert int(found.item()) == 0
    c_ref = O.gemm(gq.qT, O.E5M2, hq.qT, O.E4M3FN, gq.sc.inv, hq.sc.inv)
    ii, jj = every(H, Fd)
    absdot = O.gemm_absdot_at(gq.qT, O.E5M2, hq.qT, O.E4M3FN, gq.sc.inv, hq.sc.inv, ii, jj)
    nw = check_gemm_values(c.reshape(-1), c_ref.reshape(-1), absdot, T, None, "down wgrad fp32")
    assert nw <= 1e-3
    check_unscaled_values(host_u16(gw).reshape(-1), c_ref.reshape(-1), absdot, T, LOSS_SCALE,
                          "down wgrad fp16 unscaled")


def alpha_pairs(n, seed):
    """Inverse scales as the quantizer makes them (1 / (fp8_max / amax)), kept
    where fl32(fl64(inv_a * inv_b)) and fl32(fl32(inv_a) * fl32(inv_b)) differ."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        amax = np.exp(rng.uniform(np.log(1e-3), np.log(1e2), 2))
        ia, ib = 1.0 / (448.0 / amax[0]), 1.0 / (57344.0 / amax[1])
        ref = np.float32(O.gemm_alpha(ia, ib))
        alt = np.float32(np.float32(ia) * np.float32(ib))
        if ref != alt:
            out.append((ia, ib, ref, alt))
    return out


@pytest.mark.parametrize("shape", [(128, 128, 128), (2048, 4096, 256)])
def test_gemm_alpha_rounding_on_device(shape):
    """C = acc * alpha with acc an exact power of two (a single nonzero product
    per output), so the fp32 output holds alpha's rounding bit for bit: the
    device takes alpha = fl32(inv_a * inv_b) with the product in fp64, as the
    oracle does (pinned against exact arithmetic on the CPU), and not the
    product of the fp32-rounded inverses.  Shapes for the 128 x 128 and the
    256 x 256 kernel."""
    M, N, K = shape
    one_e5 = O.encode(O.E5M2, [1.0])[0]
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    rows = np.arange(M)
    A[rows, rows % K] = O.encode(O.E4M3FN, 2.0 ** ((rows % 8) - 4.0))  # a_i = 2^(i%8 - 4)
    B[:, :] = one_e5  # every b = 1: acc[i, j] = a_i
    a_i = (2.0 ** ((rows % 8) - 4.0)).astype(np.float32)
    Ad, Bd = dev_u8(A), dev_u8(B)
    for ia, ib, ref, alt in alpha_pairs(6, M + N):
        invd = torch.tensor([ia, ib], dtype=torch.float64, device=DEV)
        C = torch.empty((M, N), dtype=torch.float32, device=DEV)
        F.fp8_gemm(Ad, F.E4M3FN, Bd, F.E5M2, invd.data_ptr(), invd.data_ptr() + 8, C, F.OUT_F32)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        want = (a_i * ref)[:, None]  # a power of two times alpha: exact
        assert np.array_equal(got.view(np.uint32), np.broadcast_to(want, (M, N)).view(np.uint32))
        assert not np.array_equal(got[:, :1], (a_i * alt)[:, None])


@pytest.mark.parametrize("M,N", [(4096, 4096), (4000, 4112)])
def test_empty_contraction_at_large_tile_sizes(M, N):
    """Kc == 0 where the tile count would pick the 256 x 256 kernel: C = 0 * alpha
    (+0) through fp8_gemm (every output type), fp8_gemm_rowwise and
    fp8_gemm_unscale (found_inf untouched)."""
    A = torch.empty((M, 0), dtype=torch.uint8, device=DEV)
    B = torch.empty((N, 0), dtype=torch.uint8, device=DEV)
    inv = torch.tensor([0.37, 1.5], dtype=torch.float64, device=DEV)
    for out, dt in ((F.OUT_F32, torch.float32), (F.OUT_BF16, torch.bfloat16), (F.OUT_F16, torch.float16)):
        C = torch.full((M, N), 7.0, dtype=dt, device=DEV)
        F.fp8_gemm(A, F.E4M3FN, B, F.E4M3FN, inv.data_ptr(), inv.data_ptr() + 8, C, out)
        torch.cuda.synchronize()
        assert torch.count_nonzero(C.view(torch.int16 if dt != torch.float32 else torch.int32)) == 0
    inv_a = torch.full((M,), 0.25, dtype=torch.float64, device=DEV)
    inv_b = torch.full((N,), 3.0, dtype=torch.float64, device=DEV)
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_rowwise(A, F.E4M3FN, B, F.E4M3FN, inv_a, inv_b, C, F.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C.view(torch.int16)) == 0
    scale = torch.tensor([1024.0], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    C = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    F.fp8_gemm_unscale(A, F.E5M2, B, F.E4M3FN, inv.data_ptr(), inv.data_ptr() + 8, scale, found, C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C.view(torch.int16)) == 0
    assert int(found.item()) == 0


@pytest.mark.parametrize("name", ["gate", "down"])
def test_mlp_layer_copy_layouts_agree(name):
    """An MLP linear at full size (gate: 8192 x 14336 x 4096; down: 8192 x 4096
    x 14336) run as the benchmark runs it -- bf16 forward, backward of the
    loss-scaled gradient with the unscale fused -- with every transposed copy,
    with the copies fp8_linear_copies picks, and with none: the codes,
    records, outputs and the non-finite flag are the same bits (the layer
    with every copy is checked against the oracle in the config tests)."""
    from workloads.configs import mlp_linear
    L = mlp_linear(name)
    M, N, K = L.M, L.N, L.K
    x = dev_bf16(L.x()).reshape(M, K)
    w = dev_bf16(L.w()).reshape(N, K)
    gy = dev_bf16(L.gy()).reshape(M, N) * 65536.0
    runs = []
    for layout in ((True, True, True), F.fp8_linear_copies(M, N, K), (False, False, False)):
        xt, wt, gt = layout
        saved = F.LinearSaved(M, N, K, x_transposed=xt, w_transposed=wt)
        ws = F.LinearBwdWs(M, N, transposed=gt)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
        gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
        scale = torch.tensor([65536.0], dtype=torch.float32, device=DEV)
        found = torch.zeros(1, dtype=torch.int32, device=DEV)
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        torch.cuda.synchronize()
        runs.append((layout, [y.view(torch.int16), gx.view(torch.int16), gw.view(torch.int16),
                              saved.x_q, saved.w_q, ws.gy_q, saved.recs[:, :32], ws.gy_sc.buf[:32],
                              found]))
    ref = runs[0][1]
    for layout, got in runs[1:]:
        for k, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), (name, layout, k)
