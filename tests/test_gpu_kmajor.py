"""GEMMs with contraction-major operands, and linear layers without transposed
copies [FP8-TRAIN §4 backward: dgrad and wgrad contract x, W and gy over
their other dimension].

fp8_gemm_kmajor reads A stored as A^T [K, M] and/or B as B^T [K, N] with LDS
transpose reads; the products and their k order are those of fp8_gemm on the
row-major codes, so every output must be the same bits as fp8_gemm's (itself
checked against the oracle in test_gpu_kernels.py and test_gpu_full_parity.py),
and a direct oracle comparison runs on top for a few shapes.  A linear layer
built without transposed copies must give the same codes, records, outputs
and gradients as one with them.
"""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
from tests.parity import check_gemm_values, decode_out
from tests.test_gpu_kernels import OUT_FMT, dev_u8, host_out, out_tensor, random_codes

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [(64, 256, 128), (144, 272, 400), (256, 64, 48),  # 128 x 128 kernel, ragged K
          (4096, 2048, 256), (4000, 2064, 400),            # 256 x 256 kernel, ragged M, N, K
          (14000, 2048, 256),                              # 224-row tiles
          (912, 13072, 400)]                               # roles swapped when both are k-major


def bits(C):
    return C.view(torch.int32 if C.dtype == torch.float32 else torch.int16)


def operands(seed, M, N, K, fa, fb, ta, tb):
    rng = np.random.default_rng(seed)
    A = random_codes(rng, fa, (M, K))
    B = random_codes(rng, fb, (N, K))
    Ad, Bd = dev_u8(A), dev_u8(B)
    As = dev_u8(np.ascontiguousarray(A.T)) if ta else Ad
    Bs = dev_u8(np.ascontiguousarray(B.T)) if tb else Bd
    return A, B, Ad, Bd, As, Bs


@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("out", [F.OUT_F32, F.OUT_BF16, F.OUT_F16])
def test_kmajor_equals_rowmajor(ta, tb, shape, out):
    M, N, K = shape
    fa, fb = F.E5M2, F.E4M3FN
    A, B, Ad, Bd, As, Bs = operands(M + 3 * N + 7 * K + 11 * ta + 13 * tb + out, M, N, K, fa, fb, ta, tb)
    inv = np.array([2.0 ** -9 / 3.0, 1.0 / 448.0 * 0.37], np.float64)
    if out == F.OUT_F16:
        inv *= 2.0 ** -16
    invd = torch.from_numpy(inv).to(DEV)
    C1, C2 = out_tensor((M, N), out), out_tensor((M, N), out)
    C2.fill_(7.0)
    F.fp8_gemm(Ad, fa, Bd, fb, invd.data_ptr(), invd.data_ptr() + 8, C1, out)
    F.fp8_gemm_kmajor(As, fa, ta, Bs, fb, tb, invd.data_ptr(), invd.data_ptr() + 8, C2, out)
    torch.cuda.synchronize()
    assert torch.equal(bits(C1), bits(C2)), (shape, ta, tb, out)


@pytest.mark.parametrize("fa,fb", [(F.E4M3FN, F.E4M3FN), (F.E5M2, F.E5M2), (F.E4M3FN, F.E5M2)])
@pytest.mark.parametrize("shape", [(144, 272, 400), (4000, 2064, 400)])
def test_kmajor_formats_match_oracle(fa, fb, shape):
    """Both operands contraction-major, the other format pairs, every output
    against the oracle (fp32 output)."""
    M, N, K = shape
    A, B, Ad, Bd, As, Bs = operands(M + N + K + 10 * fa + fb, M, N, K, fa, fb, 1, 1)
    inv = np.array([2.0 ** -9 / 3.0, 1.0 / 448.0 * 0.37], np.float64)
    invd = torch.from_numpy(inv).to(DEV)
    C = out_tensor((M, N), F.OUT_F32)
    F.fp8_gemm_kmajor(As, fa, 1, Bs, fb, 1, invd.data_ptr(), invd.data_ptr() + 8, C, F.OUT_F32)
    torch.cuda.synchronize()
    ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(M), np.arange(N), indexing="ij")]
    c_ref = O.gemm_at(A, fa, B, fb, inv[0], inv[1], ii, jj)
    absdot = O.gemm_absdot_at(A, fa, B, fb, inv[0], inv[1], ii, jj)
    got = decode_out(OUT_FMT[F.OUT_F32], host_out(C, F.OUT_F32)).reshape(M, N)[ii, jj]
    nw = check_gemm_values(got, c_ref, absdot, K, None, f"{shape} {fa}{fb} k-major")
    assert nw <= 1e-3


@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", [(144, 272, 400), (4000, 2064, 400), (912, 13072, 400)])
def test_kmajor_unscale_equals_rowmajor(ta, tb, shape):
    """The fused-unscale epilogue on contraction-major operands: the fp16
    gradients and the flag of fp8_gemm_unscale on the row-major codes."""
    M, N, K = shape
    fa, fb = F.E5M2, F.E4M3FN
    A, B, Ad, Bd, As, Bs = operands(M + N + K + ta + 2 * tb, M, N, K, fa, fb, ta, tb)
    inv = torch.tensor([2.0 ** -9 / 3.0, 0.37 / 448.0 * 2.0 ** -14], dtype=torch.float64, device=DEV)
    scale = torch.tensor([49152.0], dtype=torch.float32, device=DEV)
    f1, f2 = (torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(2))
    C1, C2 = (torch.empty((M, N), dtype=torch.float16, device=DEV) for _ in range(2))
    F.fp8_gemm_unscale(Ad, fa, Bd, fb, inv.data_ptr(), inv.data_ptr() + 8, scale, f1, C1)
    F.fp8_gemm_kmajor_unscale(As, fa, ta, Bs, fb, tb, inv.data_ptr(), inv.data_ptr() + 8, scale, f2, C2)
    torch.cuda.synchronize()
    assert torch.equal(bits(C1), bits(C2))
    assert int(f1.item()) == int(f2.item())


def run_layer(M, N, K, transposed, delayed, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).to(DEV)
    gy = (1e-4 * 65536.0 * torch.randn(M, N, generator=g)).to(torch.bfloat16).to(DEV)
    xt, wt, gt = transposed if isinstance(transposed, tuple) else (transposed,) * 3
    saved = F.LinearSaved(M, N, K, x_transposed=xt, w_transposed=wt)
    ws = F.LinearBwdWs(M, N, transposed=gt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
    gx2 = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    gw2 = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    scale = torch.tensor([65536.0], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    if delayed:
        hx, hw, hg = (torch.full((4,), v, dtype=torch.float32, device=DEV) for v in (3.0, 0.05, 2.0))
        F.fp8_scaled_linear_fwd_delayed(x, w, saved, hx, hw, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_delayed_unscale(gy, saved, ws, hg, scale, found, gx, gw)
        hists = (hx, hw, hg)
    else:
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        F.fp8_scaled_linear_bwd(gy, saved, ws, gx2, gw2, F.OUT_BF16)
        hists = ()
    torch.cuda.synchronize()
    # the records' amax and scale fields (their partial-maximum slots depend
    # on which cast kernel ran: the small layer's one-block cast writes one)
    recs = [{k: r.read()[k] for k in ("amax_bits", "scale", "inv", "scale32_bits", "inv32_bits")}
            for r in (saved.x_sc, saved.w_sc, ws.gy_sc)]
    return dict(y=y, gx=gx, gw=gw, gx2=gx2 if not delayed else None, gw2=gw2 if not delayed else None,
                x_q=saved.x_q, w_q=saved.w_q, gy_q=ws.gy_q, found=found, hists=hists, recs=recs)


LAYOUTS = [False, (False, False, True), (True, False, False), (False, True, True),
           (True, True, False)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("delayed", [False, True])
@pytest.mark.parametrize("shape", [(64, 256, 128), (1024, 1536, 768), (4096, 4096, 2048),
                                   (2048, 14336, 4096), (2048, 4096, 14336)])
def test_linear_without_transposed_copies(shape, delayed, layout):
    """Forward, backward with the fused unscale, and (dynamic) the plain bf16
    backward: identical with all transposed copies and with none or some of
    them (x_qT, w_qT, gy_qT) -- the small layer's one-block cast, the
    128 x 128 pair launch, the 256 x 256 and 224-row forms, and the
    down-projection form whose weight gradient swaps the operands' roles."""
    M, N, K = shape
    a = run_layer(M, N, K, True, delayed, M + N + K)
    b = run_layer(M, N, K, layout, delayed, M + N + K)
    assert a["recs"] == b["recs"]
    for k in ("y", "gx", "gw", "gx2", "gw2", "x_q", "w_q", "gy_q", "found"):
        if a[k] is None:
            continue
        ta, tb = a[k], b[k]
        if ta.dtype in (torch.bfloat16, torch.float16):
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), (k, shape, delayed)
    for h1, h2 in zip(a["hists"], b["hists"]):
        assert torch.equal(h1, h2)


def test_linear_copies_on_the_device():
    """The fastest layout on MI355X's 256 CUs: the weight gradient's first-slot
    operand keeps its copy (gy for the MLP block's gate/up, x = h for down,
    whose weight gradient swaps the roles); small layers keep none; the layer
    run in that layout equals the one with every copy."""
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    assert F.fp8_linear_copies(8192, 14336, 4096) == (False, False, True)
    assert F.fp8_linear_copies(8192, 4096, 14336) == (True, False, False)
    assert F.fp8_linear_copies(64, 256, 128) == (False, False, False)
    for M, N, K in ((2048, 4096, 14336), (1024, 1536, 768)):
        a = run_layer(M, N, K, True, False, M + N)
        b = run_layer(M, N, K, F.fp8_linear_copies(M, N, K), False, M + N)
        for k in ("y", "gx", "gw", "gx2", "gw2", "found"):
            ta, tb = a[k], b[k]
            if ta.dtype in (torch.bfloat16, torch.float16):
                ta, tb = ta.view(torch.int16), tb.view(torch.int16)
            assert torch.equal(ta, tb), (k, M, N, K)
