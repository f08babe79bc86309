"""GPU parity: every C-ABI entry point against the oracle on the same seeded
inputs.  Codes, amax, scales, flags and scaler state bit-exact; GEMM outputs
within the summation-order bound (tests/parity.py)."""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
import workloads as W
from tests.parity import assert_codes_equal, check_gemm_values, decode_out

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUT_FMT = {F.OUT_BF16: O.BF16, F.OUT_F16: O.F16, F.OUT_F32: None}


def dev_bf16(bits):
    bits = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def dev_f16(bits):
    bits = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16).to(DEV)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8).copy()).to(DEV)


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_out(t, out):
    if out == F.OUT_F32:
        return t.cpu().numpy()
    return host_u16(t)


def out_tensor(shape, out):
    dt = {F.OUT_BF16: torch.bfloat16, F.OUT_F16: torch.float16, F.OUT_F32: torch.float32}[out]
    return torch.empty(shape, dtype=dt, device=DEV)


def check_rec(rec: F.ScaleRec, ref: O.Scale, what=""):
    r = rec.read()
    assert r["amax_bits"] == ref.amax_bits, what
    s_ref = np.array([ref.scale, ref.inv], np.float64)
    s_got = np.array([r["scale"], r["inv"]], np.float64)
    assert np.array_equal(s_got.view(np.uint64), s_ref.view(np.uint64)) or \
        (np.isnan(s_ref).all() and np.isnan(s_got).all()), (what, s_got, s_ref)
    assert r["scale32_bits"] == int(np.array([ref.scale32], np.float32).view(np.uint32)[0]) or np.isnan(ref.scale32)
    assert r["inv32_bits"] == int(np.array([ref.inv32], np.float32).view(np.uint32)[0]) or np.isnan(ref.inv32)
    assert 1 <= r["nparts"] <= F.AMAX_PARTS


# ------------------------------------------------------------------------ amax

@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 100, 4097, 65536 * 4 + 3, (1 << 22) + 5])
def test_amax_matches_oracle(n):
    x = W.normal_bf16(31, 7, (n,), 2.0, 0.001, 50.0)
    rec = F.ScaleRec()
    F.fp8_amax(dev_bf16(x), rec)
    torch.cuda.synchronize()
    r = rec.read()
    assert r["amax_bits"] == O.amax_bits(x)
    # the same record again: nothing left over from the first call may leak in
    y = W.normal_bf16(31, 8, (n,), 0.5)
    F.fp8_amax(dev_bf16(y), rec)
    torch.cuda.synchronize()
    assert rec.read()["amax_bits"] == O.amax_bits(y)


@pytest.mark.parametrize("special", ["nan", "inf", "neg_inf", "zeros", "neg_zero_max"])
def test_amax_special_values(special):
    n = 100_003
    x = W.normal_bf16(32, 1, (n,), 1.0)
    if special == "nan":
        x[77_777] = 0x7FC1
    elif special == "inf":
        x[5] = 0x7F80
    elif special == "neg_inf":
        x[n - 1] = 0xFF80
    elif special == "zeros":
        x[:] = 0x8000
        x[::3] = 0
    else:
        x[:] = 0x8000
        x[1234] = 0xC2C8  # -100
    rec = F.ScaleRec()
    F.fp8_amax(dev_bf16(x), rec)
    torch.cuda.synchronize()
    assert rec.read()["amax_bits"] == O.amax_bits(x)


# -------------------------------------------------------------------- quantize

SHAPES = [(16, 16), (128, 128), (144, 272), (272, 144), (256, 4096), (4096, 48), (37, 53),
          (1, 1000), (1000, 1), (1, 17), (0, 16), (16, 0), (1, 5), (7, 1)]


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("with_t", [True, False])
def test_quantize_matches_oracle(fmt, shape, with_t):
    rows, cols = shape
    sigma = 1.0 if fmt == F.E4M3FN else 1e-4
    x = W.normal_bf16(33, rows * 7 + cols, shape, sigma, 0.002, 50.0)
    ref = O.to_fp8(x, fmt, with_transpose=True)
    xd = dev_bf16(x).reshape(shape)
    rec = F.ScaleRec()
    q = torch.empty(shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=DEV) if with_t else None
    F.fp8_amax(xd, rec)
    F.fp8_quantize(xd, fmt, rec, q, qT)
    torch.cuda.synchronize()
    check_rec(rec, ref.sc, str(shape))
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, f"q {shape}")
    if with_t:
        assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, f"qT {shape}")


@pytest.mark.parametrize("with_t", [True, False])
def test_quantize_reused_record(with_t):
    """One record for a large tensor (all partial-maximum slots written, large
    amax), then for small ones (a few slots): the cast takes every slot, so the
    slots past the small tensor's count must not keep the large amax."""
    rec = F.ScaleRec()
    big = W.normal_bf16(35, 1, (4096, 2048), 1.0, 0.002, 500.0)
    bd = dev_bf16(big).reshape(big.shape)
    F.fp8_amax(bd, rec)
    F.fp8_quantize(bd, F.E4M3FN, rec, torch.empty(big.shape, dtype=torch.uint8, device=DEV))
    for shape in [(256, 272), (16, 16), (0, 16)]:
        x = W.normal_bf16(35, shape[0] + 2, shape, 0.01)
        ref = O.to_fp8(x, F.E4M3FN, with_transpose=True)
        xd = dev_bf16(x).reshape(shape)
        q = torch.empty(shape, dtype=torch.uint8, device=DEV)
        qT = torch.empty(shape[::-1], dtype=torch.uint8, device=DEV) if with_t else None
        F.fp8_amax(xd, rec)
        F.fp8_quantize(xd, F.E4M3FN, rec, q, qT)
        torch.cuda.synchronize()
        check_rec(rec, ref.sc, str(shape))
        assert_codes_equal(F.E4M3FN, q.cpu().numpy(), ref.q, f"q {shape}")
        if with_t:
            assert_codes_equal(F.E4M3FN, qT.cpu().numpy(), ref.qT, f"qT {shape}")


def finite_bf16_upto(limit):
    """Every finite bf16 pattern with |x| <= limit, both signs."""
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.decode(O.BF16, allp)
    keep = np.isfinite(v) & (np.abs(v) <= limit)
    return allp[keep]


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
@pytest.mark.parametrize("amax_kind", ["unit_scale", "odd_scale", "tiny_scale"])
def test_quantize_every_bf16_value(fmt, amax_kind):
    """Every finite bf16 value through the device converter: with amax = fp8_max
    the scale is exactly 1, so codes are the converter's rounding of each bf16
    value; other amax values make fl32(x * scale32) general fp32 values."""
    fmax = O.fp8_max(fmt)
    limit = {"unit_scale": fmax, "odd_scale": 3.3e3, "tiny_scale": 1.1e-3}[amax_kind]
    x = finite_bf16_upto(limit)
    pad = (-x.size) % 16
    x = np.concatenate([x, np.zeros(pad, np.uint16)]).reshape(-1, 16)
    ref = O.to_fp8(x, fmt)
    xd = dev_bf16(x).reshape(x.shape)
    rec = F.ScaleRec()
    q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty((16, x.shape[0]), dtype=torch.uint8, device=DEV)
    F.fp8_amax(xd, rec)
    F.fp8_quantize(xd, fmt, rec, q, qT)
    torch.cuda.synchronize()
    check_rec(rec, ref.sc)
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, "all bf16 values")
    assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, "all bf16 values, transposed")


@pytest.mark.parametrize("case", ["nan_input", "inf_input", "all_zero"])
def test_quantize_special_tensors(case):
    x = W.normal_bf16(34, 1, (64, 64), 1.0)
    if case == "nan_input":
        x[3, 5] = 0x7FC0
    elif case == "inf_input":
        x[60, 1] = 0xFF80
    else:
        x[:] = 0
        x[::2, ::3] = 0x8000
    for fmt in (F.E4M3FN, F.E5M2):
        ref = O.to_fp8(x, fmt)
        xd = dev_bf16(x).reshape(x.shape)
        rec = F.ScaleRec()
        q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        qT = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        F.fp8_amax(xd, rec)
        F.fp8_quantize(xd, fmt, rec, q, qT)
        torch.cuda.synchronize()
        check_rec(rec, ref.sc, case)
        assert_codes_equal(fmt, q.cpu().numpy(), ref.q, case)
        assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, case)


# ------------------------------------------------------------------------ GEMM

def random_codes(rng, fmt, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    v = O.decode(fmt, c)
    c[~np.isfinite(v)] = 0
    return c


GEMM_SHAPES = [(16, 16, 16), (64, 256, 128), (256, 64, 64), (144, 272, 400), (272, 144, 48),
               (384, 256, 1024), (128, 128, 0), (512, 384, 4096),
               # large enough for the 256 x 256 LDS-DMA kernel, with ragged M, N and K
               (4096, 2048, 256), (4000, 2064, 400), (2064, 4000, 1040),
               # 224 x 256 tiles (their rounds over the CUs are cheaper here):
               # ragged M, N and K, and M a multiple of 224
               (4000, 4112, 400), (14000, 2048, 256), (7168, 2560, 128),
               # the operands' roles swapped (224-row tiles along N, the tile
               # written transposed): ragged M, N and K
               (912, 13072, 400)]


@pytest.mark.parametrize("fa,fb", [(F.E4M3FN, F.E4M3FN), (F.E5M2, F.E4M3FN), (F.E4M3FN, F.E5M2),
                                   (F.E5M2, F.E5M2)])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("out", [F.OUT_F32, F.OUT_BF16, F.OUT_F16])
def test_gemm_matches_oracle(fa, fb, shape, out):
    M, N, K = shape
    rng = np.random.default_rng(M * 31 + N * 7 + K + 100 * fa + 10 * fb)
    A = random_codes(rng, fa, (M, K))
    B = random_codes(rng, fb, (N, K))
    # inverse scales like the quantizer's: e5m2 codes reach 57344, so keep
    # fp16 outputs in range with small inverses
    inv = np.array([2.0 ** -9 / 3.0, 1.0 / 448.0 * 0.37], np.float64)
    if out == F.OUT_F16:
        inv *= 2.0 ** -16  # keep |C| well below the fp16 maximum
    invd = torch.from_numpy(inv).to(DEV)
    C = out_tensor((M, N), out)
    F.fp8_gemm(dev_u8(A), fa, dev_u8(B), fb, invd.data_ptr(), invd.data_ptr() + 8, C, out)
    torch.cuda.synchronize()
    got = decode_out(OUT_FMT[out], host_out(C, out))
    # every output, also on the shapes that take the 256 x 256 kernel
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.reshape(-1), jj.reshape(-1)
    c_ref = O.gemm_at(A, fa, B, fb, inv[0], inv[1], ii, jj)
    absdot = O.gemm_absdot_at(A, fa, B, fb, inv[0], inv[1], ii, jj)
    g = got.reshape(M, N)[ii, jj] if M * N else got
    check_gemm_values(g, c_ref, absdot, K, OUT_FMT[out], f"{shape} {fa}{fb} out{out}")


# 224-row tiles along M; 256 x 256 tiles; 224-row tiles along N with the
# operands' roles swapped (each with ragged edges)
@pytest.mark.parametrize("shape", [(8208, 4112, 272), (4112, 14000, 144), (4096, 14320, 144)])
@pytest.mark.parametrize("unscale", [False, True])
def test_gemm_streamed_output(shape, unscale):
    """A 16-bit output of 64 MiB or more leaves the large-tile kernel with
    non-temporal stores: ragged M and N in each of its three tilings, bf16
    output and the fp16 output with the fused unscale.  Every output against
    the oracle, the non-finite flag, and the 64 KiB after C untouched."""
    from tests.parity import check_unscaled_values
    M, N, K = shape
    fa = F.E5M2 if unscale else F.E4M3FN
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    A = random_codes(rng, fa, (M, K))
    B = random_codes(rng, F.E4M3FN, (N, K))
    inv = np.array([2.0 ** -16 / 3.0, 1.0 / 448.0 * 0.37], np.float64)
    invd = torch.from_numpy(inv).to(DEV)
    guard = 32768
    buf = torch.full((M * N + guard,), 0x5A5A, dtype=torch.int16, device=DEV)
    if unscale:
        C = buf[:M * N].view(torch.float16).view(M, N)
        scale = torch.tensor([65536.0], dtype=torch.float32, device=DEV)
        found = torch.zeros(1, dtype=torch.int32, device=DEV)
        F.fp8_gemm_unscale(dev_u8(A), fa, dev_u8(B), F.E4M3FN, invd.data_ptr(), invd.data_ptr() + 8,
                           scale, found, C)
    else:
        C = buf[:M * N].view(torch.bfloat16).view(M, N)
        F.fp8_gemm(dev_u8(A), fa, dev_u8(B), F.E4M3FN, invd.data_ptr(), invd.data_ptr() + 8, C,
                   F.OUT_BF16)
    torch.cuda.synchronize()
    assert 2 * M * N >= 64 << 20
    assert bool(torch.all(buf[M * N:] == 0x5A5A)), "stores past C"
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.reshape(-1), jj.reshape(-1)
    c_ref = O.gemm_at(A, fa, B, F.E4M3FN, inv[0], inv[1], ii, jj)
    absdot = O.gemm_absdot_at(A, fa, B, F.E4M3FN, inv[0], inv[1], ii, jj)
    bits = buf[:M * N].cpu().numpy().view(np.uint16)
    if unscale:
        assert int(found.item()) == 0
        check_unscaled_values(bits, c_ref, absdot, K, 65536.0, f"{shape} unscaled")
    else:
        check_gemm_values(decode_out(O.BF16, bits), c_ref, absdot, K, O.BF16, f"{shape} bf16")


@pytest.mark.parametrize("shape", [(32, 48, (1 << 20) + 16), (272, 16, 65536 + 48)])
def test_gemm_long_contraction(shape):
    """A contraction of a million FP8 products (8,192 k-tiles of 128 plus a
    ragged 16): every output against the oracle's sequential fp32 sum."""
    M, N, K = shape
    rng = np.random.default_rng(K)
    A = random_codes(rng, F.E4M3FN, (M, K))
    B = random_codes(rng, F.E5M2, (N, K))
    inv = np.array([2.0 ** -9, 2.0 ** -12], np.float64)
    invd = torch.from_numpy(inv).to(DEV)
    C = out_tensor((M, N), F.OUT_F32)
    F.fp8_gemm(dev_u8(A), F.E4M3FN, dev_u8(B), F.E5M2, invd.data_ptr(), invd.data_ptr() + 8, C,
               F.OUT_F32)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(M), np.arange(N), indexing="ij")]
    c_ref = O.gemm_at(A, F.E4M3FN, B, F.E5M2, inv[0], inv[1], ii, jj)
    absdot = O.gemm_absdot_at(A, F.E4M3FN, B, F.E5M2, inv[0], inv[1], ii, jj)
    check_gemm_values(got[ii, jj], c_ref, absdot, K, OUT_FMT[F.OUT_F32], f"long K {shape}")


# ------------------------------------------------------------------ GradScaler

AMP_SIZES = [0, 1, 7, 8, 9, 8191, 8192, 8193, 70_000, 123_457]


def amp_run(grads_bits, scale_val, found0=0):
    g_dev = [dev_f16(g) for g in grads_bits]
    scale = torch.tensor([scale_val], dtype=torch.float32, device=DEV)
    found = torch.tensor([found0], dtype=torch.int32, device=DEV)
    F.amp_unscale_check(g_dev, scale, found)
    torch.cuda.synchronize()
    return [host_u16(g) for g in g_dev], int(found.item())


@pytest.mark.parametrize("scale_val", [65536.0, 3.0, 0.5, 2.0 ** 24])
def test_unscale_check_matches_oracle(scale_val):
    grads = [W.normal_f16(35, i, (n,), 1e-5 * 65536.0) for i, n in enumerate(AMP_SIZES)]
    got, found = amp_run(grads, scale_val)
    ref = [g.copy() for g in grads]
    f_ref = O.unscale_check(ref, scale_val, 0)
    assert found == f_ref
    for i, (a, b) in enumerate(zip(got, ref)):
        assert_codes_equal(O.F16, a, b, f"tensor {i} ({AMP_SIZES[i]} elements)")


@pytest.mark.parametrize("bits", [0x7C00, 0xFC00, 0x7E00])
@pytest.mark.parametrize("where", [0, 8192, 123_456])
def test_unscale_check_flags_injected_nonfinite(bits, where):
    grads = [W.normal_f16(36, i, (n,), 0.3) for i, n in enumerate(AMP_SIZES)]
    grads[-1][where] = bits
    got, found = amp_run(grads, 1024.0)
    ref = [g.copy() for g in grads]
    assert found == O.unscale_check(ref, 1024.0, 0) == 1
    for a, b in zip(got, ref):
        assert_codes_equal(O.F16, a, b)
    _, found = amp_run([grads[3]], 1024.0, found0=1)  # OR-accumulated, never cleared
    assert found == 1


def test_unscale_check_many_tensors():
    rng = np.random.default_rng(37)
    sizes = rng.integers(0, 20_000, 150)
    grads = [W.normal_f16(37, i, (int(n),), 1.0) for i, n in enumerate(sizes)]
    grads[140][int(sizes[140]) // 2] = 0x7C00 if sizes[140] else grads[140]
    got, found = amp_run(grads, 8.0)
    ref = [g.copy() for g in grads]
    assert found == O.unscale_check(ref, 8.0, 0)
    for a, b in zip(got, ref):
        assert_codes_equal(O.F16, a, b)


def test_update_scale_trajectory():
    rng = np.random.default_rng(38)
    for interval, p in ((3, 0.2), (100, 0.01), (1, 0.5)):
        scale = torch.tensor([65536.0], dtype=torch.float32, device=DEV)
        tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
        found = torch.zeros(1, dtype=torch.int32, device=DEV)
        st = O.ScalerState(np.float32(65536.0), 0)
        for step in range(300):
            f = int(rng.random() < p)
            found.fill_(f)
            F.amp_update_scale(scale, tracker, found, 2.0, 0.5, interval)
            st = O.update_scale(st, f, 2.0, 0.5, interval)
            assert float(scale.item()) == float(st.scale) or (np.isinf(st.scale) and np.isinf(scale.item()))
            assert int(tracker.item()) == st.tracker
            assert int(found.item()) == 0  # consumed and cleared


# ---------------------------------------------------------- the linear layer

def run_linear(cfg_x, cfg_w, cfg_gy, out_fwd=F.OUT_BF16, out_bwd=F.OUT_BF16):
    M, K = cfg_x.shape
    N = cfg_w.shape[0]
    x, w, gy = dev_bf16(cfg_x).reshape(M, K), dev_bf16(cfg_w).reshape(N, K), dev_bf16(cfg_gy).reshape(M, N)
    saved = F.LinearSaved(M, N, K)
    ws = F.LinearBwdWs(M, N)
    y = out_tensor((M, N), out_fwd)
    gx = out_tensor((M, K), out_bwd)
    gw = out_tensor((N, K), out_bwd)
    F.fp8_scaled_linear_fwd(x, w, saved, y, out_fwd)
    F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, out_bwd)
    torch.cuda.synchronize()
    return saved, ws, y, gx, gw


def test_linear_small_layer_full():
    """B=64, K=128, N=256 FP8 linear, fwd + dgrad + wgrad, every output checked."""
    from workloads.configs import SMALL
    x, w, gy = SMALL.x(), SMALL.w(), SMALL.gy()
    saved, ws, y, gx, gw = run_linear(x, w, gy)
    fw = O.linear_fwd(x, w)
    bw = O.linear_bwd(gy, fw)
    check_rec(saved.x_sc, fw.x.sc, "x")
    check_rec(saved.w_sc, fw.w.sc, "w")
    check_rec(ws.gy_sc, bw.gy.sc, "gy")
    for got, ref, fmt in ((saved.x_q, fw.x.q, O.E4M3FN), (saved.x_qT, fw.x.qT, O.E4M3FN),
                          (saved.w_q, fw.w.q, O.E4M3FN), (saved.w_qT, fw.w.qT, O.E4M3FN),
                          (ws.gy_q, bw.gy.q, O.E5M2), (ws.gy_qT, bw.gy.qT, O.E5M2)):
        assert_codes_equal(fmt, got.cpu().numpy(), ref)
    M, N, K = SMALL.M, SMALL.N, SMALL.K
    full = lambda a, b: np.meshgrid(np.arange(a), np.arange(b), indexing="ij")
    ii, jj = [v.reshape(-1) for v in full(M, N)]
    ad = O.gemm_absdot_at(fw.x.q, O.E4M3FN, fw.w.q, O.E4M3FN, fw.x.sc.inv, fw.w.sc.inv, ii, jj)
    check_gemm_values(O.decode(O.BF16, host_u16(y)).reshape(-1), fw.c.reshape(-1), ad, K, O.BF16, "fwd")
    ii, jj = [v.reshape(-1) for v in full(M, K)]
    ad = O.gemm_absdot_at(bw.gy.q, O.E5M2, fw.w.qT, O.E4M3FN, bw.gy.sc.inv, fw.w.sc.inv, ii, jj)
    check_gemm_values(O.decode(O.BF16, host_u16(gx)).reshape(-1), bw.c_gx.reshape(-1), ad, N, O.BF16, "dgrad")
    ii, jj = [v.reshape(-1) for v in full(N, K)]
    ad = O.gemm_absdot_at(bw.gy.qT, O.E5M2, fw.x.qT, O.E4M3FN, bw.gy.sc.inv, fw.x.sc.inv, ii, jj)
    check_gemm_values(O.decode(O.BF16, host_u16(gw)).reshape(-1), bw.c_gw.reshape(-1), ad, M, O.BF16, "wgrad")


def test_small_layer_with_gradscaler_step():
    """The small layer's backward under fp16 AMP: gy carries the loss scale
    65536, the GEMMs write fp16 gradients, then one unscale/check/update step
    (growth interval 2000): codes identical to the unscaled run's, scale stays
    65536 and the tracker reaches 1."""
    from workloads.configs import SMALL, INIT_SCALE, INTERVAL
    x, w, gy = SMALL.x(), SMALL.w(), SMALL.gy()
    gy_s = W.f32_to_bf16_bits(O.decode(O.BF16, gy).astype(np.float32) * np.float32(INIT_SCALE)).reshape(gy.shape)
    saved, ws, y, gx, gw = run_linear(x, w, gy_s, F.OUT_BF16, F.OUT_F16)
    fw = O.linear_fwd(x, w)
    bw = O.linear_bwd(gy_s, fw, out_fmt=O.F16)
    bw_plain = O.linear_bwd(gy, fw)
    assert np.array_equal(bw.gy.q, bw_plain.gy.q) and bw.gy.sc.inv == bw_plain.gy.sc.inv * INIT_SCALE
    assert_codes_equal(O.E5M2, ws.gy_q.cpu().numpy(), bw.gy.q)
    M, N, K = SMALL.M, SMALL.N, SMALL.K
    # fp16 gradients against the oracle's, to the GEMM tolerance
    for got, c_ref, A, fa, B, ia, ib, kc in (
            (gx, bw.c_gx, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.sc.inv, fw.w.sc.inv, N),
            (gw, bw.c_gw, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.sc.inv, fw.x.sc.inv, M)):
        ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(c_ref.shape[0]),
                                                      np.arange(c_ref.shape[1]), indexing="ij")]
        ad = O.gemm_absdot_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
        check_gemm_values(O.decode(O.F16, host_u16(got)).reshape(-1), c_ref.reshape(-1), ad, kc,
                          O.F16, "fp16 grad")
    # the GradScaler step on exactly those fp16 bits: bit-exact
    g_host = [host_u16(t).copy() for t in (gx, gw)]
    scale = torch.tensor([INIT_SCALE], dtype=torch.float32, device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.amp_unscale_check([gx, gw], scale, found)
    found_host = int(found.item())
    F.amp_update_scale(scale, tracker, found, 2.0, 0.5, INTERVAL)
    torch.cuda.synchronize()
    f_ref = O.unscale_check(g_host, INIT_SCALE, 0)
    assert found_host == f_ref == 0
    assert_codes_equal(O.F16, host_u16(gx), g_host[0], "unscaled gx")
    assert_codes_equal(O.F16, host_u16(gw), g_host[1], "unscaled gw")
    st = O.update_scale(O.ScalerState(np.float32(INIT_SCALE), 0), f_ref, 2.0, 0.5, INTERVAL)
    assert float(scale.item()) == float(st.scale) == INIT_SCALE
    assert int(tracker.item()) == st.tracker == 1


def test_unscale_check_views_into_flat_buffer():
    """Gradients as views at arbitrary 2-byte offsets of one flat fp16 buffer
    (a gradient bucket): partial first/last vectors must be handled without
    touching the neighbours."""
    rng = np.random.default_rng(39)
    sizes = [1, 3, 7, 8, 9, 15, 17, 8191, 8193, 20000, 5, 70001]
    offs = np.concatenate([[0], np.cumsum(sizes)])
    flat_h = W.normal_f16(39, 1, (int(offs[-1]) + 3,), 4.0)
    flat_h[int(offs[5]) + 2] = 0x7E00  # NaN inside one view
    flat = dev_f16(flat_h)
    views = [flat[1 + int(offs[t]):1 + int(offs[t + 1])] for t in range(len(sizes))]
    # unscale every other view; the others and the guard elements must not change
    chosen = [v for t, v in enumerate(views) if t % 2 == 1]
    scale = torch.tensor([8.0], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.amp_unscale_check(chosen, scale, found)
    torch.cuda.synchronize()
    ref = flat_h.copy()
    f = 0
    for t in range(len(sizes)):
        if t % 2 == 1:
            seg = ref[1 + int(offs[t]):1 + int(offs[t + 1])].copy()
            f = O.unscale_check([seg], 8.0, f)
            ref[1 + int(offs[t]):1 + int(offs[t + 1])] = seg
    assert int(found.item()) == f == 1
    assert_codes_equal(O.F16, host_u16(flat), ref, "flat buffer")
