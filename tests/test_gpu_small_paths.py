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
@pytest.mark.parametrize("copies", [True, False])
def test_small_layer_paths_match_oracle(shape, fused, copies):
    """With transposed copies the small tensors take the one-block casts; without
    them a layer whose x, W and gy hold at most 64 Ki elements each runs each
    pass in one launch (the GEMM blocks reduce and cast what they need)."""
    M, N, K = shape
    x_h = W.normal_bf16(95, 0, (M, K), 1.0, 0.001, 50.0)
    w_h = W.normal_bf16(95, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(95, 2, (M, N), 1e-3 * 65536.0)
    saved = F.LinearSaved(M, N, K, transposed=copies)
    ws = F.LinearBwdWs(M, N, transposed=copies)
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
        if got is not None:
            assert_codes_equal(fmt, got.cpu().numpy(), ref, nm)
    full_check(y, fw.c, fw.x.q, O.E4M3FN, fw.w.q, fw.x.sc.inv, fw.w.sc.inv, K, O.BF16, "y")
    post = float(np.float32(1.0) / np.float32(65536.0)) if fused else 1.0
    full_check(gx, bw.c_gx.astype(np.float64) * post, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.sc.inv * post,
               fw.w.sc.inv, N, O.F16, "gx")
    full_check(gw, bw.c_gw.astype(np.float64) * post, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.sc.inv * post,
               fw.x.sc.inv, M, O.F16, "gw")
    assert int(found.item()) == 0


def run_small(M, N, K, copies, out, x_h, w_h, gy_h, unscale):
    saved = F.LinearSaved(M, N, K, transposed=copies)
    ws = F.LinearBwdWs(M, N, transposed=copies)
    odt = {F.OUT_BF16: torch.bfloat16, F.OUT_F16: torch.float16, F.OUT_F32: torch.float32}[out]
    y = torch.empty((M, N), dtype=odt, device=DEV)
    gdt = torch.float16 if unscale else odt
    gx = torch.empty((M, K), dtype=gdt, device=DEV)
    gw = torch.empty((N, K), dtype=gdt, device=DEV)
    scale = torch.tensor([3.0 * 2.0 ** 14], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.fp8_scaled_linear_fwd(dev_bf16(x_h), dev_bf16(w_h), saved, y, out)
    if unscale:
        F.fp8_scaled_linear_bwd_unscale(dev_bf16(gy_h), saved, ws, scale, found, gx, gw)
    else:
        F.fp8_scaled_linear_bwd(dev_bf16(gy_h), saved, ws, gx, gw, out)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()
    # fp64 fields compared as bit patterns (a NaN scale equals itself)
    f64 = lambda v: int(np.array([v], np.float64).view(np.uint64)[0])
    recs = [(r.read()["amax_bits"], f64(r.read()["scale"]), f64(r.read()["inv"]),
             r.read()["scale32_bits"], r.read()["inv32_bits"]) for r in (saved.x_sc, saved.w_sc, ws.gy_sc)]
    return [bits(t) for t in (y, gx, gw)] + [saved.x_q.cpu(), saved.w_q.cpu(), ws.gy_q.cpu(),
                                             found.cpu()], recs


@pytest.mark.parametrize("kind", ["normal", "inf_in_x", "nan_in_gy", "overflow"])
@pytest.mark.parametrize("out,unscale", [(F.OUT_BF16, False), (F.OUT_F32, False), (F.OUT_F16, True)])
@pytest.mark.parametrize("shape", [(64, 256, 128), (16, 16, 16), (48, 80, 112), (256, 256, 256),
                                   (128, 1040, 48), (16, 4096, 16)])
def test_one_launch_small_layer_equals_general_path(shape, out, unscale, kind):
    """The one-launch forward and backward give the codes, records, outputs and
    flag of the cast + GEMM launches bit for bit (special values included: an
    infinite x makes x's scale 0 and its codes 0 or NaN, a NaN in gy makes
    every gradient NaN, a large gradient overflows fp16 before the unscale)."""
    M, N, K = shape
    x_h = W.normal_bf16(96, 0, (M, K), 1.0, 0.001, 50.0)
    w_h = W.normal_bf16(96, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(96, 2, (M, N), 1e-3 * 65536.0)
    if kind == "inf_in_x":
        x_h = x_h.copy()
        x_h.reshape(-1)[7] = 0x7F80
    elif kind == "nan_in_gy":
        gy_h = gy_h.copy()
        gy_h.reshape(-1)[(M * N) // 3] = 0x7FC1
    elif kind == "overflow":
        gy_h = W.normal_bf16(96, 3, (M, N), 3e4)
    a, ra = run_small(M, N, K, True, out, x_h, w_h, gy_h, unscale)
    b, rb = run_small(M, N, K, False, out, x_h, w_h, gy_h, unscale)
    assert ra == rb
    for name, ta, tb in zip(("y", "gx", "gw", "x_q", "w_q", "gy_q", "found"), a, b):
        assert torch.equal(ta, tb), (name, shape, out, kind)
