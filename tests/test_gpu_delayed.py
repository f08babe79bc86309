"""GPU parity for delayed scaling (fp8_quantize_delayed and the delayed linear
entry points) against the oracle's to_fp8_delayed / linear_*_delayed: codes
and transposed codes, the scale fields taken from the history, the current
amax and the pushed history, all bit-exact, over several steps; GEMM outputs
within the bound of tests/parity.py."""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
import workloads as W
from tests.parity import assert_codes_equal, check_gemm_values
from workloads import configs as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def same(a, b):
    """Equal, or both NaN (a NaN scale has no single correct encoding)."""
    return a == b or (np.isnan(a) and np.isnan(b))


def check_step(rec, hist_dev, q_dev, qT_dev, ref, fmt, what):
    r = rec.read()
    assert r["amax_bits"] == ref.amax_bits, what
    assert same(r["scale"], ref.sc.scale) and same(r["inv"], ref.sc.inv), what
    assert same(np.float32(r["scale32"]), ref.sc.scale32), what
    assert same(np.float32(r["inv32"]), ref.sc.inv32), what
    assert np.array_equal(hist_dev.cpu().numpy().view(np.uint32), ref.hist.view(np.uint32)), what
    assert_codes_equal(fmt, q_dev.cpu().numpy().reshape(ref.q.shape), ref.q, what)
    if qT_dev is not None:
        assert_codes_equal(fmt, qT_dev.cpu().numpy(), ref.qT, what)


def run_steps(shape, fmt, H, steps, sigmas, transposed=True, seed=0):
    rows, cols = shape
    hist_h = np.zeros(H, np.float32)
    x0 = W.normal_bf16(seed, 0, shape, sigmas[0])
    hist_h[0] = O.bits_to_f32(O.amax_bits(x0))
    hist = torch.from_numpy(hist_h.copy()).to(DEV)
    rec = F.ScaleRec(device=DEV)
    q = torch.empty(shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=DEV) if transposed else None
    for t in range(steps):
        x = W.normal_bf16(seed, t + 1, shape, sigmas[t % len(sigmas)])
        F.fp8_quantize_delayed(dev16(x), fmt, rec, hist, q, qT)
        torch.cuda.synchronize()
        ref = O.to_fp8_delayed(x, fmt, hist_h, with_transpose=transposed)
        check_step(rec, hist, q, qT, ref, fmt, f"{shape} fmt {fmt} H {H} step {t}")
        hist_h = ref.hist


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
@pytest.mark.parametrize("H", [1, 4, 16])
def test_delayed_tiled_sequence(fmt, H):
    run_steps((256, 384), fmt, H, 5, [1.0, 4.0, 0.25, 100.0])


@pytest.mark.parametrize("shape", [(48, 80), (16, 16), (4096, 4096)])
def test_delayed_shapes(shape):
    run_steps(shape, O.E4M3FN, 8, 3, [1.0, 2.0])


def test_delayed_more_tiles_than_partial_slots():
    # 8192 x 4096 is 2048 tiles of 128 x 128: 1024 blocks, two tiles each
    run_steps((8192, 4096), O.E5M2, 4, 2, [1e-4, 3e-4])


@pytest.mark.parametrize("shape", [(1, 1000), (37, 61), (8, 24)])
def test_delayed_flat_and_ragged(shape):
    run_steps(shape, O.E4M3FN, 3, 3, [1.0, 0.5], transposed=False)
    run_steps(shape, O.E5M2, 3, 2, [1.0, 0.5], transposed=shape[1] % 16 != 0 or shape[0] % 16 != 0)


def test_delayed_max_history_and_specials():
    H = F.MAX_HISTORY
    hist_h = (np.arange(H, dtype=np.float32) + 1.0) / 64.0
    hist_h[700] = 1e6  # the largest entry sits deep in the history
    x = W.normal_bf16(9, 1, (64, 128), 1.0)
    x[3, 5] = 0x7F80  # +inf: saturates at the scale from the history
    hist = torch.from_numpy(hist_h.copy()).to(DEV)
    rec = F.ScaleRec(device=DEV)
    q = torch.empty((64, 128), dtype=torch.uint8, device=DEV)
    qT = torch.empty((128, 64), dtype=torch.uint8, device=DEV)
    F.fp8_quantize_delayed(dev16(x), O.E4M3FN, rec, hist, q, qT)
    torch.cuda.synchronize()
    ref = O.to_fp8_delayed(x, O.E4M3FN, hist_h)
    check_step(rec, hist, q, qT, ref, O.E4M3FN, "max history")
    # a NaN entry makes the scale NaN and every code NaN
    hist_h = ref.hist.copy()
    hist_h[5] = np.nan
    hist = torch.from_numpy(hist_h.copy()).to(DEV)
    F.fp8_quantize_delayed(dev16(x), O.E4M3FN, rec, hist, q, qT)
    torch.cuda.synchronize()
    ref = O.to_fp8_delayed(x, O.E4M3FN, hist_h)
    check_step(rec, hist, q, qT, ref, O.E4M3FN, "nan history")


def test_delayed_linear_steps():
    """Three training steps of a 512 x 768 x 384 layer with delayed scaling on
    x, W and gy: every code, scale field, history and output against the
    oracle."""
    M, N, K, H = 512, 768, 384, 4
    saved = F.LinearSaved(M, N, K, device=DEV)
    ws = F.LinearBwdWs(M, N, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    hx, hw, hg = (np.full(H, v, np.float32) for v in (4.0, 0.1, 1e-3))
    dhx, dhw, dhg = (torch.from_numpy(h.copy()).to(DEV) for h in (hx, hw, hg))
    for t in range(3):
        x = W.normal_bf16(50 + t, 0, (M, K), 1.0 + t)
        w = W.normal_bf16(50 + t, 1, (N, K), 0.02)
        gy = W.normal_bf16(50 + t, 2, (M, N), 1e-4)
        F.fp8_scaled_linear_fwd_delayed(dev16(x), dev16(w), saved, dhx, dhw, y)
        F.fp8_scaled_linear_bwd_delayed(dev16(gy), saved, ws, dhg, gx, gw)
        torch.cuda.synchronize()
        fw, hx, hw = O.linear_fwd_delayed(x, w, hx, hw)
        bw, hg = O.linear_bwd_delayed(gy, fw, hg)
        check_step(saved.x_sc, dhx, saved.x_q, saved.x_qT, fw.x, O.E4M3FN, f"x step {t}")
        check_step(saved.w_sc, dhw, saved.w_q, saved.w_qT, fw.w, O.E4M3FN, f"w step {t}")
        check_step(ws.gy_sc, dhg, ws.gy_q, ws.gy_qT, bw.gy, O.E5M2, f"gy step {t}")
        full = lambda a, b: [v.reshape(-1) for v in np.meshgrid(np.arange(a), np.arange(b),
                                                                 indexing="ij")]
        for got, c_ref, A, fa, B, ia, ib, kc, what in (
                (y, fw.c, fw.x.q, O.E4M3FN, fw.w.q, fw.x.sc.inv, fw.w.sc.inv, K, "fwd"),
                (gx, bw.c_gx, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.sc.inv, fw.w.sc.inv, N, "dgrad"),
                (gw, bw.c_gw, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.sc.inv, fw.x.sc.inv, M, "wgrad")):
            ii, jj = full(*c_ref.shape)
            ad = O.gemm_absdot_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
            check_gemm_values(O.decode(O.BF16, host_u16(got)).reshape(-1), c_ref.reshape(-1), ad,
                              kc, O.BF16, f"{what} step {t}")


def test_delayed_at_the_quantize_workload_size():
    """The 2^28-element activation tensor of the quantize-path workload, e4m3,
    one delayed step after a history seeded with a quarter of its amax (so
    part of the tensor saturates)."""
    x = C.quant_act()
    a = O.bits_to_f32(O.amax_bits(x))
    hist_h = np.array([a / 4, a / 8], np.float32)
    hist = torch.from_numpy(hist_h.copy()).to(DEV)
    rec = F.ScaleRec(device=DEV)
    q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    F.fp8_quantize_delayed(dev16(x), O.E4M3FN, rec, hist, q)
    torch.cuda.synchronize()
    ref = O.to_fp8_delayed(x, O.E4M3FN, hist_h, with_transpose=False)
    check_step(rec, hist, q, None, ref, O.E4M3FN, "2^28")


@pytest.mark.parametrize("transposed", [True, False])
def test_delayed_record_reused_after_a_larger_tensor(transposed):
    """A record whose partial slots a larger tensor filled (all 1024, large
    amax), then delayed casts of small tensors (a few slots): the amax pushed
    to the history takes every slot, so the ones past the small cast's block
    count must not keep the large tensor's maxima."""
    rec = F.ScaleRec(device=DEV)
    big = W.normal_bf16(41, 0, (4096, 2048), 1.0, 0.002, 500.0)
    F.fp8_amax(dev16(big).reshape(big.shape), rec)
    shape = (272, 144)
    hist_h = np.full(4, 0.5, np.float32)
    hist = torch.from_numpy(hist_h.copy()).to(DEV)
    q = torch.empty(shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty(shape[::-1], dtype=torch.uint8, device=DEV) if transposed else None
    for t in range(3):
        x = W.normal_bf16(41, t + 1, shape, 0.01)
        F.fp8_quantize_delayed(dev16(x).reshape(shape), O.E4M3FN, rec, hist, q, qT)
        torch.cuda.synchronize()
        ref = O.to_fp8_delayed(x, O.E4M3FN, hist_h, with_transpose=transposed)
        check_step(rec, hist, q, qT, ref, O.E4M3FN, f"reused record, step {t}")
        hist_h = ref.hist


@pytest.mark.parametrize("shape,transposed", [((4224, 4096), True), ((4099, 4097), False)])
def test_delayed_two_level_over_stale_slots(shape, transposed):
    """Tensors that need more blocks than there are partial slots (1056 tiles
    of 128 x 128; 2050 flat blocks with a ragged tail) take the two-level
    cast, whose blocks fold their maxima into slots cleared first: a record
    whose slots a tensor of larger amax filled must not leak into the amax
    pushed to the history."""
    rec = F.ScaleRec(device=DEV)
    big = W.normal_bf16(43, 0, (4096, 2048), 1.0, 0.002, 500.0)
    F.fp8_amax(dev16(big).reshape(big.shape), rec)
    hist_h = np.array([0.004, 0.002], np.float32)
    hist = torch.from_numpy(hist_h.copy()).to(DEV)
    rows, cols = shape
    q = torch.empty(shape, dtype=torch.uint8, device=DEV)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=DEV) if transposed else None
    for t in range(2):
        x = W.normal_bf16(43, t + 1, shape, 1e-3)
        F.fp8_quantize_delayed(dev16(x).reshape(shape), O.E5M2, rec, hist, q, qT)
        torch.cuda.synchronize()
        ref = O.to_fp8_delayed(x, O.E5M2, hist_h, with_transpose=transposed)
        check_step(rec, hist, q, qT, ref, O.E5M2, f"two-level {shape}, step {t}")
        hist_h = ref.hist


@pytest.mark.parametrize("copies", [True, False])
def test_delayed_linear_two_level_casts(copies):
    """A layer whose x, W and gy each need more cast blocks than a record has
    partial slots (4224 x 4352 x 4096: 1056, 1088 and 1122 tiles), so x and W
    share one two-level launch (slot clear, one pass per block, atomic slot
    maxima) and gy takes another; two steps with delayed scaling: codes,
    scale fields, histories against the oracle bit for bit, GEMM outputs
    sampled."""
    M, N, K, H = 4224, 4352, 4096, 4
    saved = F.LinearSaved(M, N, K, device=DEV, transposed=copies)
    ws = F.LinearBwdWs(M, N, device=DEV, transposed=copies)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    hx, hw, hg = (np.full(H, v, np.float32) for v in (3.0, 0.08, 4e-4))
    dhx, dhw, dhg = (torch.from_numpy(h.copy()).to(DEV) for h in (hx, hw, hg))
    rng = np.random.default_rng(7)
    for t in range(2):
        x = W.normal_bf16(60 + t, 0, (M, K), 1.0 + t)
        w = W.normal_bf16(60 + t, 1, (N, K), 0.02)
        gy = W.normal_bf16(60 + t, 2, (M, N), 1e-4)
        F.fp8_scaled_linear_fwd_delayed(dev16(x), dev16(w), saved, dhx, dhw, y)
        F.fp8_scaled_linear_bwd_delayed(dev16(gy), saved, ws, dhg, gx, gw)
        torch.cuda.synchronize()
        # the oracle's delayed casts (its composite linear functions would also
        # run the three full GEMMs on the CPU)
        xq = O.to_fp8_delayed(x, O.E4M3FN, hx)
        wq = O.to_fp8_delayed(w, O.E4M3FN, hw)
        gq = O.to_fp8_delayed(gy, O.E5M2, hg)
        hx, hw, hg = xq.hist, wq.hist, gq.hist
        check_step(saved.x_sc, dhx, saved.x_q, saved.x_qT, xq, O.E4M3FN, f"x step {t}")
        check_step(saved.w_sc, dhw, saved.w_q, saved.w_qT, wq, O.E4M3FN, f"w step {t}")
        check_step(ws.gy_sc, dhg, ws.gy_q, ws.gy_qT, gq, O.E5M2, f"gy step {t}")
        for got, A, fa, B, ia, ib, kc, what in (
                (y, xq.q, O.E4M3FN, wq.q, xq.sc.inv, wq.sc.inv, K, "fwd"),
                (gx, gq.q, O.E5M2, wq.qT, gq.sc.inv, wq.sc.inv, N, "dgrad"),
                (gw, gq.qT, O.E5M2, xq.qT, gq.sc.inv, xq.sc.inv, M, "wgrad")):
            R, C = got.shape
            ii, jj = rng.integers(0, R, 2048), rng.integers(0, C, 2048)
            c_ref = O.gemm_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
            ad = O.gemm_absdot_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
            check_gemm_values(O.decode(O.BF16, host_u16(got)[ii, jj]), c_ref, ad, kc, O.BF16,
                              f"{what} step {t}")
