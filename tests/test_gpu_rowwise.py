"""GPU parity of row-wise scaling ["FP8训练：量化、自动微分、Torchao", §1: one
scale per row, carried through the accumulation]: fp8_quantize_rowwise
(codes, transposed codes, amax and inverse-scale vectors bit-exact against the
oracle's to_fp8_rowwise), fp8_gemm_rowwise (within the summation-order bound of
tests/parity.py, with the per-element factor fl32(inv_a[m] * inv_b[n])) and
the row-wise linear forward/backward."""
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


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8).copy()).to(DEV)


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_out(t, out):
    return t.cpu().numpy() if out == F.OUT_F32 else host_u16(t)


def out_tensor(shape, out):
    dt = {F.OUT_BF16: torch.bfloat16, F.OUT_F16: torch.float16, F.OUT_F32: torch.float32}[out]
    return torch.empty(shape, dtype=dt, device=DEV)


def row_mag_bf16(seed, rows, cols, lo10, hi10, axis=0):
    """Normal values whose rows (axis 0) or columns (axis 1) have magnitudes
    spread log-uniformly over 10^lo10 .. 10^hi10: the case row-wise scaling
    is for."""
    z = W.normal_f32(seed, 0, rows * cols, 1.0).reshape(rows, cols).astype(np.float64)
    n = rows if axis == 0 else cols
    mags = 10.0 ** (lo10 + (hi10 - lo10) * W.uniform(seed, 1, n))
    f = z * (mags[:, None] if axis == 0 else mags[None, :])
    return W.f32_to_bf16_bits(f.astype(np.float32)).reshape(rows, cols)


def check_vec(amax, inv, ref: O.RowScales, what):
    a = amax.cpu().numpy().view(np.uint32)
    assert np.array_equal(a, ref.amax_bits), f"{what}: amax differs at " \
        f"{np.nonzero(a != ref.amax_bits)[0][:5]}"
    i = inv.cpu().numpy()
    same = (i.view(np.uint64) == ref.inv.view(np.uint64)) | (np.isnan(i) & np.isnan(ref.inv))
    assert same.all(), f"{what}: inverse scales differ at {np.nonzero(~same)[0][:5]}"


def run_quant(x_h, fmt, with_t=True):
    rows, cols = x_h.shape
    x = dev_bf16(x_h) if x_h.size else torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    rs = F.RowScalesDev(rows)
    cs = F.RowScalesDev(cols) if with_t else None
    q = torch.full((rows, cols), 0x5A, dtype=torch.uint8, device=DEV)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=DEV) if with_t else None
    # stale contents must not leak into the result
    rs.amax.fill_(123.0)
    if cs is not None:
        cs.amax.fill_(-7.0)
    F.fp8_quantize_rowwise(x, fmt, rs, q, cs, qT)
    torch.cuda.synchronize()
    return rs, cs, q, qT


# the partial maxima live in q's memory: the thinnest shapes leave the least room
QUANT_SHAPES = [(16, 16), (128, 128), (144, 272), (272, 144), (400, 48), (48, 1040), (1040, 528),
                (16, 2064), (2064, 16)]


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
@pytest.mark.parametrize("shape", QUANT_SHAPES)
@pytest.mark.parametrize("with_t", [True, False])
def test_quantize_rowwise_matches_oracle(fmt, shape, with_t):
    rows, cols = shape
    x_h = row_mag_bf16(rows * 7 + cols, rows, cols, -6, 3)
    rs, cs, q, qT = run_quant(x_h, fmt, with_t)
    ref = O.to_fp8_rowwise(x_h, fmt, with_transpose=with_t)
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, f"q {shape}")
    check_vec(rs.amax, rs.inv, ref.rows, f"rows {shape}")
    if with_t:
        assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, f"qT {shape}")
        check_vec(cs.amax, cs.inv, ref.cols, f"cols {shape}")


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
def test_quantize_rowwise_column_magnitudes(fmt):
    """Magnitudes spread along columns: the column scales of the transposed
    copy are the ones that matter."""
    x_h = row_mag_bf16(91, 272, 400, -5, 2, axis=1)
    rs, cs, q, qT = run_quant(x_h, fmt)
    ref = O.to_fp8_rowwise(x_h, fmt)
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, "q")
    assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, "qT")
    check_vec(rs.amax, rs.inv, ref.rows, "rows")
    check_vec(cs.amax, cs.inv, ref.cols, "cols")


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
def test_quantize_rowwise_special_rows(fmt):
    """A row of zeros (scale of amax 0), a row with +inf, one with NaN, one of
    negative zeros and subnormal bf16 values, one at the bf16 maximum."""
    x_h = row_mag_bf16(92, 160, 144, -2, 2)
    x_h[3] = 0
    x_h[17, 5] = 0x7F80          # +inf
    x_h[40, 100] = 0xFFC1        # a NaN with payload
    x_h[41] = 0x8000             # -0
    x_h[41, ::3] = 0x0001        # smallest subnormal
    x_h[130] = 0x7F7F            # bf16 max
    x_h[131, 7] = 0xFF80         # -inf
    rs, cs, q, qT = run_quant(x_h, fmt)
    ref = O.to_fp8_rowwise(x_h, fmt)
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, "q")
    assert_codes_equal(fmt, qT.cpu().numpy(), ref.qT, "qT")
    check_vec(rs.amax, rs.inv, ref.rows, "rows")
    check_vec(cs.amax, cs.inv, ref.cols, "cols")


@pytest.mark.parametrize("shape", [(0, 32), (32, 0), (0, 0)])
def test_quantize_rowwise_empty(shape):
    rows, cols = shape
    x_h = np.zeros(shape, np.uint16)
    rs, cs, q, qT = run_quant(x_h, F.E4M3FN)
    ref = O.to_fp8_rowwise(x_h, O.E4M3FN)
    check_vec(rs.amax, rs.inv, ref.rows, "rows")
    check_vec(cs.amax, cs.inv, ref.cols, "cols")


def random_codes(rng, fmt, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[~np.isfinite(O.decode(fmt, c))] = 0
    return c


RW_GEMM_SHAPES = [(16, 16, 16), (144, 272, 400), (272, 144, 48), (128, 128, 0), (512, 384, 4096),
                  # 256 x 256 kernel, ragged M, N and K
                  (4096, 2048, 256), (4000, 2064, 400)]


@pytest.mark.parametrize("fa,fb", [(F.E4M3FN, F.E4M3FN), (F.E5M2, F.E4M3FN)])
@pytest.mark.parametrize("shape", RW_GEMM_SHAPES)
@pytest.mark.parametrize("out", [F.OUT_F32, F.OUT_BF16, F.OUT_F16])
def test_gemm_rowwise_matches_oracle(fa, fb, shape, out):
    M, N, K = shape
    rng = np.random.default_rng(M * 13 + N * 5 + K + 100 * fa + 7 * out)
    A = random_codes(rng, fa, (M, K))
    B = random_codes(rng, fb, (N, K))
    # inverse scales as a row-wise cast of rows spanning 10^-6 .. 10^3 gives
    ia = (10.0 ** rng.uniform(-6, 3, M)) / 448.0
    ib = (10.0 ** rng.uniform(-3, 0, N)) / (448.0 if fb == F.E4M3FN else 57344.0)
    if out == F.OUT_F16:
        ia *= 2.0 ** -14  # keep |C| below the fp16 maximum
    C = out_tensor((M, N), out)
    F.fp8_gemm_rowwise(dev_u8(A), fa, dev_u8(B), fb, torch.from_numpy(ia).to(DEV),
                       torch.from_numpy(ib).to(DEV), C, out)
    torch.cuda.synchronize()
    got = decode_out(OUT_FMT[out], host_out(C, out)).reshape(M, N)
    if M * N * K <= (1 << 26):
        ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(M), np.arange(N), indexing="ij")]
    else:
        ii, jj = rng.integers(0, M, 4000), rng.integers(0, N, 4000)
    c_ref = O.gemm_vec_at(A, fa, B, fb, ia, ib, ii, jj)
    absdot = O.gemm_absdot_vec_at(A, fa, B, fb, ia, ib, ii, jj)
    check_gemm_values(got[ii, jj], c_ref, absdot, K, OUT_FMT[out], f"{shape} {fa}{fb} out{out}")


def run_linear_rw(x_h, w_h, gy_h, out=F.OUT_BF16):
    M, K = x_h.shape
    N = w_h.shape[0]
    saved = F.LinearSavedRW(M, N, K)
    ws = F.LinearBwdWsRW(M, N)
    y, gx, gw = out_tensor((M, N), out), out_tensor((M, K), out), out_tensor((N, K), out)
    F.fp8_scaled_linear_fwd_rowwise(dev_bf16(x_h), dev_bf16(w_h), saved, y, out)
    F.fp8_scaled_linear_bwd_rowwise(dev_bf16(gy_h), saved, ws, gx, gw, out)
    torch.cuda.synchronize()
    return saved, ws, y, gx, gw


def check_linear_rw(x_h, w_h, gy_h, out, n_pts=None, seed=0):
    M, K = x_h.shape
    N = w_h.shape[0]
    saved, ws, y, gx, gw = run_linear_rw(x_h, w_h, gy_h, out)
    fw = O.linear_fwd_rowwise(x_h, w_h)
    bw = O.linear_bwd_rowwise(gy_h, fw)
    for got, ref, fmt, what in ((saved.x_q, fw.x.q, O.E4M3FN, "x_q"), (saved.x_qT, fw.x.qT, O.E4M3FN, "x_qT"),
                                (saved.w_q, fw.w.q, O.E4M3FN, "w_q"), (saved.w_qT, fw.w.qT, O.E4M3FN, "w_qT"),
                                (ws.gy_q, bw.gy.q, O.E5M2, "gy_q"), (ws.gy_qT, bw.gy.qT, O.E5M2, "gy_qT")):
        assert_codes_equal(fmt, got.cpu().numpy(), ref, what)
    check_vec(saved.x_row_amax, saved.x_row_inv, fw.x.rows, "x rows")
    check_vec(saved.x_col_amax, saved.x_col_inv, fw.x.cols, "x cols")
    check_vec(saved.w_row_amax, saved.w_row_inv, fw.w.rows, "w rows")
    check_vec(saved.w_col_amax, saved.w_col_inv, fw.w.cols, "w cols")
    check_vec(ws.gy_row_amax, ws.gy_row_inv, bw.gy.rows, "gy rows")
    check_vec(ws.gy_col_amax, ws.gy_col_inv, bw.gy.cols, "gy cols")
    rng = np.random.default_rng(seed)
    for got, A, fa, B, ia, ib, Kc, what in (
            (y, fw.x.q, O.E4M3FN, fw.w.q, fw.x.rows.inv, fw.w.rows.inv, K, "y"),
            (gx, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.rows.inv, fw.w.cols.inv, N, "gx"),
            (gw, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.cols.inv, fw.x.cols.inv, M, "gw")):
        R, Cn = got.shape
        if n_pts is None:
            ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(R), np.arange(Cn), indexing="ij")]
        else:
            ii, jj = rng.integers(0, R, n_pts), rng.integers(0, Cn, n_pts)
        c_ref = O.gemm_vec_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
        absdot = O.gemm_absdot_vec_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
        g = decode_out(OUT_FMT[out], host_out(got, out)).reshape(R, Cn)[ii, jj]
        check_gemm_values(g, c_ref, absdot, Kc, OUT_FMT[out], what)


@pytest.mark.parametrize("out", [F.OUT_BF16, F.OUT_F32])
def test_linear_rowwise_matches_oracle(out):
    M, N, K = 272, 400, 144
    x_h = row_mag_bf16(93, M, K, -4, 2)
    w_h = row_mag_bf16(94, N, K, -3, -1)
    gy_h = row_mag_bf16(95, M, N, -8, -3)
    check_linear_rw(x_h, w_h, gy_h, out)


def test_linear_rowwise_large_sampled():
    """A 2048 x 1536 x 1024 layer (256 x 256 kernel for every GEMM), outputs
    sampled."""
    M, N, K = 2048, 1536, 1024
    x_h = row_mag_bf16(96, M, K, -3, 1)
    w_h = W.normal_bf16(96, 5, (N, K), 0.02)
    gy_h = row_mag_bf16(97, M, N, -7, -4)
    check_linear_rw(x_h, w_h, gy_h, F.OUT_BF16, n_pts=3000, seed=1)
