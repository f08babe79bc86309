"""GPU tests of the PyTorch integration (fp8_scaled_gemm_amd.nn): Float8Linear
forward/backward through autograd against the oracle's FP8 linear, delayed
scaling histories over several steps, and the GradScaler wrapper's
skip/backoff/growth behaviour and gradient norm against the oracle."""
import numpy as np
import pytest
import torch
from torch import nn

import fp8_scaled_gemm_amd as F
import fp8_scaled_gemm_amd.nn as FN
import oracle as O
import workloads as W
from tests.parity import assert_codes_equal, check_gemm_values

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits, requires_grad=False):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)
    return t.requires_grad_(requires_grad)


def host_u16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_out(got, c_ref, A, fa, B, ia, ib, K, what):
    ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(c_ref.shape[0]),
                                                  np.arange(c_ref.shape[1]), indexing="ij")]
    ad = O.gemm_absdot_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
    check_gemm_values(O.decode(O.BF16, host_u16(got)).reshape(-1), c_ref.reshape(-1), ad, K,
                      O.BF16, what)


@pytest.mark.parametrize("B,T,K,N", [(2, 64, 128, 256), (2, 1024, 2048, 4096)])
def test_float8_linear_autograd_matches_oracle(B, T, K, N):
    """The small layer (each pass one launch, no transposed copies) and a layer
    whose weight gradient takes the large-tile kernel (only gy's transposed
    copy kept, x and W read contraction-major), every output against the
    oracle through autograd."""
    x_h = W.normal_bf16(61, 0, (B * T, K), 1.0)
    w_h = W.normal_bf16(61, 1, (N, K), 0.02)
    gy_h = W.normal_bf16(61, 2, (B * T, N), 1e-3)
    lin = nn.Linear(K, N, bias=False, dtype=torch.bfloat16, device=DEV)
    with torch.no_grad():
        lin.weight.copy_(dev_bf16(w_h))
    f8 = FN.Float8Linear.from_float(lin)
    x = dev_bf16(x_h).reshape(B, T, K).requires_grad_(True)
    y = f8(x)
    assert y.shape == (B, T, N) and y.dtype == torch.bfloat16
    # the autograd node keeps FP8 codes and scale records only, no bf16 input
    node = y.grad_fn
    while node is not None and "ScaledLinear" not in type(node).__name__ and \
            "scaled_linear" not in type(node).__name__:
        node = node.next_functions[0][0] if node.next_functions else None
    assert node is not None, "no FP8 linear node in the graph"
    saved = node.saved_tensors
    assert len(saved) == 5 and all(t.dtype == torch.uint8 for t in saved)
    xt, wt, _ = F.fp8_linear_copies(B * T, N, K)
    assert (saved[1].numel() > 0, saved[3].numel() > 0) == (xt, wt)
    y.backward(dev_bf16(gy_h).reshape(B, T, N))
    torch.cuda.synchronize()
    fw = O.linear_fwd(x_h, w_h)
    bw = O.linear_bwd(gy_h, fw)
    check_out(y.reshape(B * T, N), fw.c, fw.x.q, O.E4M3FN, fw.w.q, fw.x.sc.inv, fw.w.sc.inv, K, "y")
    check_out(x.grad.reshape(B * T, K), bw.c_gx, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.sc.inv,
              fw.w.sc.inv, N, "gx")
    check_out(lin.weight.grad, bw.c_gw, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.sc.inv, fw.x.sc.inv,
              B * T, "gw")
    assert f8.weight.grad is lin.weight.grad  # one shared parameter


def test_float8_linear_delayed_steps_match_oracle():
    M, K, N, H = 128, 256, 128, 4
    lin = nn.Linear(K, N, bias=False, dtype=torch.bfloat16, device=DEV)
    w_h = W.normal_bf16(62, 1, (N, K), 0.02)
    with torch.no_grad():
        lin.weight.copy_(dev_bf16(w_h))
    f8 = FN.Float8Linear.from_float(lin, scaling="delayed", history_len=H)
    hx = hw = hg = None
    for t in range(3):
        x_h = W.normal_bf16(62, 10 + t, (M, K), 1.0 + 3 * t)
        gy_h = W.normal_bf16(62, 20 + t, (M, N), 1e-3 * (t + 1))
        x = dev_bf16(x_h, requires_grad=True)
        y = f8(x)
        y.backward(dev_bf16(gy_h))
        torch.cuda.synchronize()
        if t == 0:  # the module seeds each history with the first tensor's amax
            seed = lambda a: np.array([O.bits_to_f32(O.amax_bits(a))] + [0.0] * (H - 1), np.float32)
            hx, hw, hg = seed(x_h), seed(w_h), seed(gy_h)
        fw, hx, hw = O.linear_fwd_delayed(x_h, w_h, hx, hw)
        bw, hg = O.linear_bwd_delayed(gy_h, fw, hg)
        for got, ref in ((f8.hist_x, hx), (f8.hist_w, hw), (f8.hist_gy, hg)):
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32)), t
        check_out(y, fw.c, fw.x.q, O.E4M3FN, fw.w.q, fw.x.sc.inv, fw.w.sc.inv, K, f"y {t}")
        check_out(x.grad, bw.c_gx, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.sc.inv, fw.w.sc.inv, N,
                  f"gx {t}")
        lin.weight.grad = None


def test_float8_linear_rowwise_autograd_matches_oracle():
    M, K, N = 192, 160, 272
    rng_rows = lambda seed, r, c, lo, hi: W.f32_to_bf16_bits(
        (W.normal_f32(seed, 0, r * c, 1.0).reshape(r, c) *
         (10.0 ** (lo + (hi - lo) * W.uniform(seed, 1, r)))[:, None]).astype(np.float32)).reshape(r, c)
    x_h = rng_rows(63, M, K, -3, 2)
    w_h = W.normal_bf16(63, 5, (N, K), 0.02)
    gy_h = rng_rows(64, M, N, -6, -2)
    lin = nn.Linear(K, N, bias=False, dtype=torch.bfloat16, device=DEV)
    with torch.no_grad():
        lin.weight.copy_(dev_bf16(w_h))
    f8 = FN.Float8Linear.from_float(lin, scaling="rowwise")
    x = dev_bf16(x_h, requires_grad=True)
    y = f8(x)
    node = y.grad_fn.next_functions[0][0]
    # codes (4) and the amax / inverse-scale vectors (8): no bf16 input kept
    assert len(node.saved_tensors) == 12
    assert all(t.dtype in (torch.uint8, torch.float32, torch.float64) for t in node.saved_tensors)
    y.backward(dev_bf16(gy_h))
    torch.cuda.synchronize()
    fw = O.linear_fwd_rowwise(x_h, w_h)
    bw = O.linear_bwd_rowwise(gy_h, fw)
    for got, ref, A, fa, B, ia, ib, Kc, what in (
            (y, fw.c, fw.x.q, O.E4M3FN, fw.w.q, fw.x.rows.inv, fw.w.rows.inv, K, "y"),
            (x.grad, bw.c_gx, bw.gy.q, O.E5M2, fw.w.qT, bw.gy.rows.inv, fw.w.cols.inv, N, "gx"),
            (lin.weight.grad, bw.c_gw, bw.gy.qT, O.E5M2, fw.x.qT, bw.gy.cols.inv, fw.x.cols.inv, M,
             "gw")):
        ii, jj = [v.reshape(-1) for v in np.meshgrid(np.arange(ref.shape[0]),
                                                      np.arange(ref.shape[1]), indexing="ij")]
        ad = O.gemm_absdot_vec_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
        check_gemm_values(O.decode(O.BF16, host_u16(got)).reshape(-1), ref.reshape(-1), ad, Kc,
                          O.BF16, what)


@pytest.mark.parametrize("scaling", FN.SCALINGS)
def test_converted_mlp_block_trains(scaling):
    """A SwiGLU block converted by convert_to_float8_training: forward and
    backward run through the FP8 kernels (the gating itself is torch), and
    stay within FP8 quantization error of the bf16 block."""
    torch.manual_seed(0)
    T, H, Fd = 256, 128, 384

    class MLP(nn.Module):
        def __init__(self):
            super().__init__()
            self.gate = nn.Linear(H, Fd, bias=False, dtype=torch.bfloat16)
            self.up = nn.Linear(H, Fd, bias=False, dtype=torch.bfloat16)
            self.down = nn.Linear(Fd, H, bias=False, dtype=torch.bfloat16)

        def forward(self, x):
            return self.down(torch.nn.functional.silu(self.gate(x)) * self.up(x))

    ref = MLP().to(DEV)
    for p in ref.parameters():
        nn.init.normal_(p, 0.0, 0.05)
    f8 = MLP().to(DEV)
    f8.load_state_dict(ref.state_dict())
    FN.convert_to_float8_training(f8, scaling=scaling)
    assert all(isinstance(getattr(f8, n), FN.Float8Linear) for n in ("gate", "up", "down"))
    x = torch.randn(T, H, device=DEV, dtype=torch.bfloat16)
    y_ref, y8 = ref(x.float().bfloat16()), f8(x)
    rel = (y8.float() - y_ref.float()).norm() / y_ref.float().norm()
    assert rel < 0.1, rel
    y8.float().pow(2).mean().backward()
    y_ref.float().pow(2).mean().backward()
    for n in ("gate", "up", "down"):
        g8, gr = getattr(f8, n).weight.grad.float(), getattr(ref, n).weight.grad.float()
        assert torch.isfinite(g8).all()
        assert (g8 - gr).norm() / gr.norm() < 0.2, n


def test_grad_scaler_skip_backoff_growth_and_norm():
    ps = [nn.Parameter(torch.zeros(n, dtype=torch.float16, device=DEV)) for n in (4096, 777, 64)]
    opt = torch.optim.SGD(ps, lr=1.0)
    sc = FN.GradScaler(init_scale=1024.0, growth_interval=2)
    st = O.ScalerState(np.float32(1024.0), 0)
    for step in range(6):
        grads = [W.normal_f16(70 + step, i, (p.numel(),), 1e-2 * float(st.scale))
                 for i, p in enumerate(ps)]
        if step == 3:
            grads[1][5] = 0x7C00  # +inf in one gradient
        for p, g in zip(ps, grads):
            p.grad = torch.from_numpy(g.view(np.int16)).view(torch.float16).to(DEV)
        before = [p.detach().clone() for p in ps]
        norm = sc.unscale_(opt, with_norm=True)
        sc.step(opt)
        ref = [g.copy() for g in grads]
        found = O.unscale_check(ref, st.scale)
        for p, r in zip(ps, ref):
            assert np.array_equal(host_u16(p.grad), r)  # unscaled in place, bit-exact
        s_ref, n_ref = O.grad_norm(ref)
        n_got = norm.cpu().numpy().astype(np.float64)
        if found:
            assert not np.isfinite(n_got[1])
            assert all(torch.equal(p, b) for p, b in zip(ps, before))  # step skipped
        else:
            assert abs(n_got[1] - n_ref) <= 11 * 2.0 ** -24 * n_ref + 1e-12
            assert not all(torch.equal(p, b) for p, b in zip(ps, before))
        sc.update()
        st = O.update_scale(st, found, 2.0, 0.5, 2)
        assert sc.state() == (float(st.scale), st.tracker, 0), step
        for p in ps:
            p.grad = None


def test_float8_linear_under_torch_compile_matches_eager():
    """The dynamic-scaling linear is a registered operator with a fake
    implementation, so torch.compile (dynamo + AOT autograd, fullgraph) keeps
    it as one opaque call: a two-layer MLP compiled and eager give the same
    outputs and gradients bit for bit."""
    torch.manual_seed(0)
    K, F_, T = 128, 256, 96

    class Mlp(nn.Module):
        def __init__(self):
            super().__init__()
            self.up = nn.Linear(K, F_, bias=False, dtype=torch.bfloat16, device=DEV)
            self.down = nn.Linear(F_, K, bias=False, dtype=torch.bfloat16, device=DEV)

        def forward(self, x):
            return self.down(torch.nn.functional.gelu(self.up(x)))

    eager = FN.convert_to_float8_training(Mlp())
    comp = FN.convert_to_float8_training(Mlp())
    with torch.no_grad():
        for a, b in zip(eager.parameters(), comp.parameters()):
            b.copy_(a)
    cm = torch.compile(comp, backend="aot_eager", fullgraph=True)
    x = torch.randn(T, K, dtype=torch.bfloat16, device=DEV)
    gy = torch.randn(T, K, dtype=torch.bfloat16, device=DEV) * 1e-2
    xe, xc = x.clone().requires_grad_(True), x.clone().requires_grad_(True)
    ye, yc = eager(xe), cm(xc)
    ye.backward(gy)
    yc.backward(gy)
    torch.cuda.synchronize()
    assert torch.equal(ye.view(torch.int16), yc.view(torch.int16))
    assert torch.equal(xe.grad.view(torch.int16), xc.grad.view(torch.int16))
    for a, b in zip(eager.parameters(), comp.parameters()):
        assert torch.equal(a.grad.view(torch.int16), b.grad.view(torch.int16))


def test_backward_scratch_is_kept_across_steps():
    lin = nn.Linear(128, 256, bias=False, dtype=torch.bfloat16, device=DEV)
    f8 = FN.Float8Linear.from_float(lin, scaling="delayed")
    ids = []
    for _ in range(3):
        x = torch.randn(64, 128, dtype=torch.bfloat16, device=DEV, requires_grad=True)
        f8(x).backward(torch.randn(64, 256, dtype=torch.bfloat16, device=DEV))
        ids.append(id(f8._ws[1]))
    assert len(set(ids)) == 1


def dev_f16(bits, requires_grad=False):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)
    return t.requires_grad_(requires_grad)


def test_fp16_float8_linear_with_grad_scaler_matches_oracle():
    """An fp16 layer under loss scaling [PT-CH20 §20.2.2]: fp16 x and W cast
    by the fp16-input kernels, fp16 y; the output gradient carries the loss
    scale S, the input gradient keeps it, the weight gradient leaves the wgrad
    GEMM unscaled and checked with the attached scaler's scale, and the
    scaler's unscale_ leaves that gradient alone.  Every output against the
    oracle's composition."""
    from tests.parity import check_unscaled_values
    M, K, N, S = 192, 256, 160, 1024.0
    x_h = W.normal_f16(91, 1, (M, K), 1.0)
    w_h = W.normal_f16(91, 2, (N, K), 0.02)
    gy_h = W.normal_f16(91, 3, (M, N), 1e-3 * S)   # carries the loss scale
    lin = nn.Linear(K, N, bias=False, dtype=torch.float16, device=DEV)
    with torch.no_grad():
        lin.weight.copy_(dev_f16(w_h))
    scaler = FN.GradScaler(init_scale=S, device=DEV)
    f8 = FN.Float8Linear.from_float(lin).attach_grad_scaler(scaler)
    x = dev_f16(x_h, requires_grad=True)
    y = f8(x)
    assert y.dtype == torch.float16
    y.backward(dev_f16(gy_h))
    torch.cuda.synchronize()
    xq = O.to_fp8(x_h, O.E4M3FN, in_fmt=O.F16)
    wq = O.to_fp8(w_h, O.E4M3FN, in_fmt=O.F16)
    gq = O.to_fp8(gy_h, O.E5M2, in_fmt=O.F16)
    full = lambda a, b: [v.reshape(-1) for v in np.meshgrid(np.arange(a), np.arange(b), indexing="ij")]
    # y: fp16 forward output
    ii, jj = full(M, N)
    c = O.gemm(xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv)
    ad = O.gemm_absdot_at(xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, ii, jj)
    check_gemm_values(O.decode(O.F16, host_u16(y)).reshape(-1), c.reshape(-1), ad, K, O.F16, "y")
    # gx: fp16, still carrying S
    ii, jj = full(M, K)
    c = O.gemm(gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv)
    ad = O.gemm_absdot_at(gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv, ii, jj)
    check_gemm_values(O.decode(O.F16, host_u16(x.grad)).reshape(-1), c.reshape(-1), ad, N, O.F16,
                      "gx")
    # gW: unscaled by S in the epilogue
    ii, jj = full(N, K)
    c = O.gemm(gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.sc.inv, xq.sc.inv)
    ad = O.gemm_absdot_at(gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.sc.inv, xq.sc.inv, ii, jj)
    gw_bits = host_u16(lin.weight.grad).copy()
    check_unscaled_values(gw_bits, c, ad, M, S, "gW")
    # the scaler: no non-finite value, unscale_ leaves the layer's gradient alone
    opt = torch.optim.SGD([lin.weight], lr=0.0)
    scaler.unscale_(opt)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(lin.weight.grad), gw_bits)
    assert scaler.state()[2] == 0
    scaler.step(opt)
    scaler.update()
    assert scaler.state()[:2] == (S, 1)


def test_fp16_two_layer_model_skips_on_overflow():
    """A two-layer fp16 model converted with a GradScaler: a loss scale that
    overflows an fp16 weight gradient sets the flag in the wgrad epilogue, the
    optimizer step is skipped, the scale halves; with a sane scale the next step
    is taken."""
    torch.manual_seed(3)
    K, F_, T = 128, 256, 64
    model = nn.Sequential(nn.Linear(K, F_, bias=False), nn.ReLU(),
                          nn.Linear(F_, K, bias=False)).to(DEV, torch.float16)
    scaler = FN.GradScaler(init_scale=2.0 ** 30, device=DEV)
    FN.convert_to_float8_training(model, grad_scaler=scaler)
    assert all(isinstance(m, FN.Float8Linear) and m.grad_scaler is scaler
               for m in (model[0], model[2]))
    opt = torch.optim.SGD(model.parameters(), lr=1e-2)
    x = torch.randn(T, K, dtype=torch.float16, device=DEV)
    before = [p.detach().clone() for p in model.parameters()]
    loss = model(x).float().square().mean()
    scaler.scale(loss).backward()
    scaler.step(opt)
    torch.cuda.synchronize()
    assert scaler.state()[2] == 1  # overflow seen
    assert all(torch.equal(a, b) for a, b in zip(before, model.parameters()))  # step skipped
    scaler.update()
    assert scaler.get_scale() == 2.0 ** 29
    # a scale that keeps the gradients finite: the step is taken
    scaler._scale.fill_(256.0)
    opt.zero_grad(set_to_none=True)
    loss = model(x).float().square().mean()
    scaler.scale(loss).backward()
    scaler.step(opt)
    torch.cuda.synchronize()
    assert scaler.state()[2] == 0
    scaler.update()
    assert any(not torch.equal(a, b) for a, b in zip(before, model.parameters()))


@pytest.mark.parametrize("M,N,K", [(64, 256, 128), (512, 768, 1024), (2048, 4096, 14336)])
def test_linear_records_need_no_initialisation(M, N, K):
    """The layer's op allocates its scale records without zeroing them: the
    forward and the backward write every field they read.  The linear entry
    points with records first filled with 0xFF bytes (NaN and garbage in every
    field and partial slot) give the same outputs and record fields, bit for
    bit, as with zeroed records: on the one-launch small path (64 x 256 x 128),
    the general path, and a size whose backward keeps a transposed copy."""
    g = torch.Generator(device="cpu").manual_seed(M + N + K)
    x = (torch.randn(M, K, generator=g)).to(torch.bfloat16).to(DEV)
    w = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    gy = (torch.randn(M, N, generator=g) * 1e-4).to(torch.bfloat16).to(DEV)
    xt, wt, gt = F.fp8_linear_copies(M, N, K)
    runs = []
    for fill in (0x00, 0xFF):
        recs = torch.full((2, F.SCALE_REC_BYTES), fill, dtype=torch.uint8, device=DEV)
        saved = F.LinearSaved(M, N, K, x_transposed=xt, w_transposed=wt)
        saved = F.LinearSaved(M, N, K, tensors=(saved.x_q, saved.x_qT, saved.w_q, saved.w_qT, recs))
        gy_rec = F.ScaleRec(buf=torch.full((F.SCALE_REC_BYTES,), fill, dtype=torch.uint8, device=DEV))
        ws = F.LinearBwdWs(M, N, transposed=gt, gy_sc=gy_rec)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        gx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
        gw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, F.OUT_BF16)
        torch.cuda.synchronize()
        runs.append([y.view(torch.int16), gx.view(torch.int16), gw.view(torch.int16), saved.x_q,
                     saved.w_q, ws.gy_q, recs[:, :32], gy_rec.buf[:32]])
    for k, (a, b) in enumerate(zip(*runs)):
        assert torch.equal(a, b), (M, N, K, k)
