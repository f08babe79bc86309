"""GPU parity at the five workloads' full sizes, through the same C-ABI calls
bench.py times.  FP8 codes (row-major and transposed), amax, scales, non-finite
flags and scaler state are compared in full, bit-exact; GEMM outputs at
sampled coordinates, each computed by the oracle one by one, within the bound
of tests/parity.py."""
import time

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


def log(msg):
    print(f"[configs {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def dev16(bits, dtype=torch.bfloat16):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(dtype).to(DEV)


def host16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_rec(rec, sc, what):
    r = rec.read()
    assert r["amax_bits"] == sc.amax_bits, what
    assert r["scale"] == sc.scale and r["inv"] == sc.inv, what
    assert np.float32(r["scale32"]) == sc.scale32 and np.float32(r["inv32"]) == sc.inv32, what


def sampled_gemm_check(got_dev, out_fmt, A, fa, B, fb, inv_a, inv_b, n_pts, seed, what):
    M, N = got_dev.shape
    rng = np.random.default_rng(seed)
    ii = rng.integers(0, M, n_pts)
    jj = rng.integers(0, N, n_pts)
    # always include the corners (first/last tile, ragged edges)
    ii = np.concatenate([ii, [0, M - 1, 0, M - 1]])
    jj = np.concatenate([jj, [0, N - 1, N - 1, 0]])
    c_ref = O.gemm_at(A, fa, B, fb, inv_a, inv_b, ii, jj)
    ad = O.gemm_absdot_at(A, fa, B, fb, inv_a, inv_b, ii, jj)
    got = host16(got_dev)[ii, jj]
    return check_gemm_values(O.decode(out_fmt, got), c_ref, ad, A.shape[1], out_fmt, what)


def run_and_check_linear(x_h, w_h, gy_h, out_bwd, n_pts, seed, what, xq_ref=None):
    """fwd (bf16 y) + bwd through the C ABI; every code and scale against the
    oracle, GEMM outputs sampled.  Returns device gradients and the oracle
    quantizations (so a caller can reuse a shared input's)."""
    M, K = x_h.shape
    N = w_h.shape[0]
    x, w, gy = dev16(x_h), dev16(w_h), dev16(gy_h)
    saved = F.LinearSaved(M, N, K)
    ws = F.LinearBwdWs(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gdt = torch.float16 if out_bwd == F.OUT_F16 else torch.bfloat16
    gx = torch.empty((M, K), dtype=gdt, device=DEV)
    gw = torch.empty((N, K), dtype=gdt, device=DEV)
    log(f"{what}: GPU fwd+bwd M={M} N={N} K={K}")
    F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
    F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, out_bwd)
    torch.cuda.synchronize()
    log(f"{what}: oracle quantize")
    xq = xq_ref if xq_ref is not None else O.to_fp8(x_h, O.E4M3FN)
    wq = O.to_fp8(w_h, O.E4M3FN)
    gq = O.to_fp8(gy_h, O.E5M2)
    for rec, sc, nm in ((saved.x_sc, xq.sc, "x"), (saved.w_sc, wq.sc, "W"), (ws.gy_sc, gq.sc, "gy")):
        check_rec(rec, sc, f"{what} {nm}")
    for got, ref, fmt, nm in ((saved.x_q, xq.q, O.E4M3FN, "x_q"), (saved.x_qT, xq.qT, O.E4M3FN, "x_qT"),
                              (saved.w_q, wq.q, O.E4M3FN, "w_q"), (saved.w_qT, wq.qT, O.E4M3FN, "w_qT"),
                              (ws.gy_q, gq.q, O.E5M2, "gy_q"), (ws.gy_qT, gq.qT, O.E5M2, "gy_qT")):
        assert_codes_equal(fmt, got.cpu().numpy(), ref, f"{what} {nm}")
    log(f"{what}: sampled GEMM outputs")
    ofmt = O.F16 if out_bwd == F.OUT_F16 else O.BF16
    sampled_gemm_check(y, O.BF16, xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, n_pts,
                       seed, f"{what} fwd")
    sampled_gemm_check(gx, ofmt, gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv, n_pts,
                       seed + 1, f"{what} dgrad")
    sampled_gemm_check(gw, ofmt, gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.sc.inv, xq.sc.inv, n_pts,
                       seed + 2, f"{what} wgrad")
    return gx, gw, xq


def test_square_layer_with_gradscaler_step():
    """4096^3 layer exactly as bench.py runs it: bf16 forward, fp16 backward of
    the loss-scaled gradient, then one unscale/check/update step."""
    cfg = C.SQUARE
    x_h, w_h, gy_h = cfg.x(), cfg.w(), cfg.gy()
    gy_s = W.f32_to_bf16_bits(O.decode(O.BF16, gy_h).astype(np.float32) *
                              np.float32(C.INIT_SCALE)).reshape(gy_h.shape)
    gx, gw, _ = run_and_check_linear(x_h, w_h, gy_s, F.OUT_F16, 2048, 20, "square")
    g_host = [host16(gx), host16(gw)]
    scale = torch.tensor([C.INIT_SCALE], dtype=torch.float32, device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.amp_unscale_check([gx, gw], scale, found)
    f_gpu = int(found.item())
    F.amp_update_scale(scale, tracker, found, C.GROWTH, C.BACKOFF, C.INTERVAL)
    torch.cuda.synchronize()
    f_ref = O.unscale_check(g_host, C.INIT_SCALE, 0)
    assert f_gpu == f_ref
    assert_codes_equal(O.F16, host16(gx), g_host[0], "unscaled gx")
    assert_codes_equal(O.F16, host16(gw), g_host[1], "unscaled gW")
    st = O.update_scale(O.ScalerState(np.float32(C.INIT_SCALE), 0), f_ref, C.GROWTH, C.BACKOFF,
                        C.INTERVAL)
    assert float(scale.item()) == float(st.scale) and int(tracker.item()) == st.tracker


def test_mlp_block_three_linears():
    """Transformer MLP block, tokens 8192, hidden 4096, ffn 14336: gate and up
    ([14336,4096], sharing x) and down ([4096,14336]), forward and backward."""
    xq_shared = None
    for k, name in enumerate(("gate", "up", "down")):
        lin = C.mlp_linear(name)
        log(f"generating {lin.name}")
        x_h, w_h, gy_h = lin.x(), lin.w(), lin.gy()
        reuse = xq_shared if name == "up" else None
        _, _, xq = run_and_check_linear(x_h, w_h, gy_h, F.OUT_BF16, 512, 30 + 3 * k, name, reuse)
        if name == "gate":
            xq_shared = xq
        del x_h, w_h, gy_h
        torch.cuda.empty_cache()


def test_shared_input_linear_is_the_full_linear():
    """The MLP block's up projection on gate's cast of x (bench.py's direct
    path: W_up alone is reduced and cast, its GEMM reads gate's x codes, its
    backward gate's transposed x codes and record) gives the same bits as a
    full fp8_scaled_linear_fwd/bwd of (x, W_up)."""
    M, K, N = 512, 1024, 768
    x = dev16(W.normal_bf16(91, 0, (M, K), 1.0))
    wg = dev16(W.normal_bf16(91, 1, (N, K), 0.02))
    wu = dev16(W.normal_bf16(91, 2, (N, K), 0.02))
    gy = dev16(W.normal_bf16(91, 3, (M, N), 1e-4))
    bf = dict(dtype=torch.bfloat16, device=DEV)
    outs = []
    for shared in (False, True):
        y, gx, gw = torch.empty(M, N, **bf), torch.empty(M, K, **bf), torch.empty(N, K, **bf)
        ws = F.LinearBwdWs(M, N)
        if shared:
            sg = F.LinearSaved(M, N, K)
            F.fp8_scaled_linear_fwd(x, wg, sg, torch.empty(M, N, **bf))
            own = F.LinearSaved(M, N, K)
            su = F.LinearSaved(M, N, K, tensors=(sg.x_q, sg.x_qT, own.w_q, own.w_qT, own.recs))
            su.x_sc = sg.x_sc
            F.fp8_amax(wu, su.w_sc)
            F.fp8_quantize(wu, F.E4M3FN, su.w_sc, su.w_q, su.w_qT)
            F.fp8_gemm(su.x_q, F.E4M3FN, su.w_q, F.E4M3FN, su.x_sc.inv_ptr(), su.w_sc.inv_ptr(),
                       y, F.OUT_BF16)
        else:
            su = F.LinearSaved(M, N, K)
            F.fp8_scaled_linear_fwd(x, wu, su, y)
        F.fp8_scaled_linear_bwd(gy, su, ws, gx, gw)
        torch.cuda.synchronize()
        outs.append([host16(t) for t in (y, gx, gw)])
    for a, b, nm in zip(outs[0], outs[1], ("y", "gx", "gW")):
        assert np.array_equal(a, b), nm


@pytest.mark.parametrize("which", ["activations_e4m3", "gradients_e5m2"])
def test_quantize_pass_2pow28(which):
    """amax + scale + quantize-cast of a 268,435,456-element bf16 tensor:
    magnitudes 10^U(-6,3) to e4m3, and 10^U(-8,-2) to e5m2."""
    if which == "activations_e4m3":
        x_h, fmt = C.quant_act(), F.E4M3FN
    else:
        x_h, fmt = C.quant_grad(), F.E5M2
    x = dev16(x_h)
    rec = F.ScaleRec()
    q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    log(f"{which}: GPU amax + quantize")
    F.fp8_amax(x, rec)
    F.fp8_quantize(x, fmt, rec, q)
    torch.cuda.synchronize()
    log(f"{which}: oracle")
    ref = O.to_fp8(x_h, fmt, with_transpose=False)
    check_rec(rec, ref.sc, which)
    assert_codes_equal(fmt, q.cpu().numpy(), ref.q, which)


@pytest.mark.parametrize("rowwise", [False, True])
def test_quantize_transposed_streaming_size(rowwise):
    """The cast with its transposed copy at a size that streams from HBM
    (16400 x 16400, 1.08 GB moved): ragged edge tiles and 129^2 = 16641 tiles,
    not a multiple of the 8 XCDs the streaming block order splits them over."""
    side = 16400
    x_h = W.normal_bf16(36, 1, (side, side), 1.0, 0.001, 50.0)
    x = dev16(x_h).reshape(side, side)
    q = torch.empty((side, side), dtype=torch.uint8, device=DEV)
    qT = torch.empty((side, side), dtype=torch.uint8, device=DEV)
    log(f"rowwise={rowwise}: GPU cast")
    if rowwise:
        rs, cs = F.RowScalesDev(side), F.RowScalesDev(side)
        F.fp8_quantize_rowwise(x, F.E4M3FN, rs, q, cs, qT)
    else:
        rec = F.ScaleRec()
        F.fp8_amax(x, rec)
        F.fp8_quantize(x, F.E4M3FN, rec, q, qT)
    torch.cuda.synchronize()
    log(f"rowwise={rowwise}: oracle")
    if rowwise:
        ref = O.to_fp8_rowwise(x_h, F.E4M3FN)
        for got, want, nm in ((rs, ref.rows, "rows"), (cs, ref.cols, "cols")):
            assert np.array_equal(got.amax.cpu().numpy().view(np.uint32), want.amax_bits), nm
            assert np.array_equal(got.inv.cpu().numpy().view(np.uint64), want.inv.view(np.uint64)), nm
    else:
        ref = O.to_fp8(x_h, F.E4M3FN, with_transpose=True)
        check_rec(rec, ref.sc, "per-tensor")
    assert_codes_equal(F.E4M3FN, q.cpu().numpy(), ref.q, "q")
    assert_codes_equal(F.E4M3FN, qT.cpu().numpy(), ref.qT, "qT")


@pytest.mark.parametrize("delayed", [False, True])
def test_quantize_flat_past_one_pass_per_block(delayed):
    """A flat cast of 2^29 + 13 elements: more 16-byte vectors than the flat
    kernel's one-pass blocks cover, so blocks stride (dynamic: 65,536 blocks;
    delayed: 1,024), plus a 5-element tail.  Codes and record bit-exact."""
    n = (1 << 29) + 13
    x_h = W.logmag_bf16(87, 0, (n,), -4.0, 2.0)
    x = dev16(x_h)
    rec = F.ScaleRec()
    q = torch.empty(n, dtype=torch.uint8, device=DEV)
    log(f"flat cast n={n} delayed={delayed}: GPU")
    if delayed:
        hist = torch.full((4,), 37.0, dtype=torch.float32, device=DEV)
        F.fp8_quantize_delayed(x, F.E4M3FN, rec, hist, q)
    else:
        F.fp8_amax(x, rec)
        F.fp8_quantize(x, F.E4M3FN, rec, q)
    torch.cuda.synchronize()
    log("oracle")
    if delayed:
        ref = O.to_fp8_delayed(x_h, O.E4M3FN, np.full(4, 37.0, np.float32), with_transpose=False)
        r = rec.read()
        assert r["amax_bits"] == ref.amax_bits  # the current amax, pushed to the history
        assert r["scale"] == ref.sc.scale and r["inv"] == ref.sc.inv
        assert np.array_equal(hist.cpu().numpy(), ref.hist)
        ref_q = ref.q
    else:
        ref = O.to_fp8(x_h, O.E4M3FN, with_transpose=False)
        check_rec(rec, ref.sc, "flat")
        ref_q = ref.q
    assert_codes_equal(O.E4M3FN, q.cpu().numpy(), ref_q, "flat striding")


def _scaler_reference(pristine_h, injections):
    """The oracle's trajectory: per step the scale it runs with, and after its
    update (found, scale, tracker).  A step's flag is the oracle's
    unscale_check of that step's data at that scale: the resident tensors
    (whose flag depends only on the scale, so it is computed once per
    distinct scale, tensor by tensor) and, on an injected step, the injected
    tensor with its inf/NaN."""
    inj = {j.step: j for j in injections}
    st = O.ScalerState(np.float32(C.INIT_SCALE), 0)
    base = {}
    before, traj = [], []
    for s in range(C.SCALER_STEPS):
        sc = float(st.scale)
        if sc not in base:
            f = 0
            for g in pristine_h:
                f = O.unscale_check([g.copy()], sc, f)
            base[sc] = f
        found = base[sc]
        if s in inj:
            g = pristine_h[inj[s].tensor].copy()
            g[inj[s].index] = inj[s].bits
            found = O.unscale_check([g], sc, found)
        before.append(sc)
        st = O.update_scale(st, found, C.GROWTH, C.BACKOFF, C.SCALER_INTERVAL)
        traj.append((found, float(st.scale), st.tracker))
    return before, traj


def test_gradscaler_200_tensors_1000_steps_full_size():
    """200 fp16 gradients (sizes log-uniform 4K..64M, ~1.7e9 elements), 1000
    steps with an inf/NaN injected into a random tensor with probability 0.01,
    growth interval 100.  Each step restores the tensors from a resident copy
    (values N(0,1e-5) * 65536), injects per the schedule, then runs one
    amp_unscale_check over all 200 tensors and amp_update_scale.  The
    found/scale/tracker trajectory must equal the oracle's over all 1000 steps
    (the oracle runs unscale_check on every step's data, see
    _scaler_reference); the unscaled values are compared in full at the first
    step that runs with each distinct scale, and sampled (with the injected
    element) at the first injected and the last step."""
    sizes = C.scaler_sizes()
    injections = C.injection_schedule(sizes)
    log(f"scaler: {len(sizes)} tensors, {int(sizes.sum())} elements, {len(injections)} injections")
    pristine_h = [C.scaler_grad(t, int(n), C.INIT_SCALE) for t, n in enumerate(sizes)]
    log("scaler: oracle trajectory")
    before, traj = _scaler_reference(pristine_h, injections)
    full_at = {}
    for s, sc in enumerate(before):
        full_at.setdefault(sc, s)
    full_steps = set(full_at.values())
    pristine = [dev16(g, torch.float16) for g in pristine_h]
    work = [torch.empty_like(p) for p in pristine]
    scale = torch.tensor([C.INIT_SCALE], dtype=torch.float32, device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    hist = torch.zeros((C.SCALER_STEPS, 3), dtype=torch.float64, device=DEV)
    inj = {j.step: j for j in injections}
    first_inj = injections[0].step if injections else None
    inj_bits = torch.tensor([0], dtype=torch.int16, device=DEV)
    for s in range(C.SCALER_STEPS):
        for wv, pv in zip(work, pristine):
            wv.copy_(pv)
        if s in inj:
            j = inj[s]
            inj_bits.fill_(int(np.array([j.bits], np.uint16).view(np.int16)[0]))
            work[j.tensor].view(torch.int16)[j.index:j.index + 1].copy_(inj_bits)
        F.amp_unscale_check(work, scale, found)
        hist[s, 0].copy_(found[0])
        F.amp_update_scale(scale, tracker, found, C.GROWTH, C.BACKOFF, C.SCALER_INTERVAL)
        hist[s, 1].copy_(scale[0])
        hist[s, 2].copy_(tracker[0])
        if s in full_steps:
            torch.cuda.synchronize()
            log(f"scaler: full element-wise check at step {s} (scale {before[s]})")
            for t, wv in enumerate(work):
                ref = pristine_h[t].copy()
                if s in inj and inj[s].tensor == t:
                    ref[inj[s].index] = inj[s].bits
                O.unscale_check([ref], before[s], 0)
                assert_codes_equal(O.F16, host16(wv), ref, f"step {s} tensor {t}")
            del ref
        elif s in (first_inj, C.SCALER_STEPS - 1):
            torch.cuda.synchronize()
            log(f"scaler: sampled check at step {s}")
            rng = np.random.default_rng(s)
            for t in rng.choice(len(sizes), 20, replace=False).tolist() + \
                    ([inj[s].tensor] if s in inj else []):
                n = int(sizes[t])
                idx = np.unique(np.concatenate([rng.integers(0, n, 5000),
                                                [inj[s].index] if (s in inj and inj[s].tensor == t) else []]).astype(np.int64))
                src = pristine_h[t][idx].copy()
                if s in inj and inj[s].tensor == t:
                    src[np.searchsorted(idx, inj[s].index)] = inj[s].bits
                O.unscale_check([src], before[s], 0)
                got = host16(work[t])[idx]
                assert_codes_equal(O.F16, got, src, f"step {s} tensor {t}")
        if s % 100 == 0:
            log(f"scaler: step {s}")
    torch.cuda.synchronize()
    h = hist.cpu().numpy()
    assert sum(f for f, _, _ in traj) == len(injections)
    for s in range(C.SCALER_STEPS):
        assert (int(h[s, 0]), float(h[s, 1]), int(h[s, 2])) == traj[s], f"step {s}"
    log(f"scaler: trajectory ok, final scale {traj[-1][1]}, tracker {traj[-1][2]}")


def test_gradscaler_downsized_every_step_elementwise():
    """The same run on 200 tensors of 4K..64K elements, values regenerated every
    step as fp16(N(0,1e-5) * scale_t), compared element by element with the
    oracle at every one of the 1000 steps."""
    sizes = C.scaler_sizes(lo=4096, hi=65536)
    injections = C.injection_schedule(sizes)
    inj = {j.step: j for j in injections}
    scale = torch.tensor([C.INIT_SCALE], dtype=torch.float32, device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    st = O.ScalerState(np.float32(C.INIT_SCALE), 0)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    flat_dev = torch.empty(int(offs[-1]), dtype=torch.float16, device=DEV)
    views = [flat_dev[int(offs[t]):int(offs[t + 1])] for t in range(len(sizes))]
    for s in range(C.SCALER_STEPS):
        cur = float(st.scale)
        g = np.concatenate([C.scaler_grad(t, int(n), cur, step=s) for t, n in enumerate(sizes)])
        if s in inj:
            g[int(offs[inj[s].tensor]) + inj[s].index] = inj[s].bits
        flat_dev.copy_(torch.from_numpy(g.view(np.int16)).view(torch.float16).to(DEV))
        F.amp_unscale_check(views, scale, found)
        f_gpu = int(found.item())
        F.amp_update_scale(scale, tracker, found, C.GROWTH, C.BACKOFF, C.SCALER_INTERVAL)
        ref = [g[int(offs[t]):int(offs[t + 1])].copy() for t in range(len(sizes))]
        f_ref = O.unscale_check(ref, cur, 0)
        assert f_gpu == f_ref == (1 if s in inj else 0), f"step {s}"
        assert_codes_equal(O.F16, host16(flat_dev), np.concatenate(ref), f"step {s}")
        st = O.update_scale(st, f_ref, C.GROWTH, C.BACKOFF, C.SCALER_INTERVAL)
        assert float(scale.item()) == float(st.scale) and int(tracker.item()) == st.tracker
        if s % 200 == 0:
            log(f"downsized scaler: step {s}, scale {float(st.scale)}")


# ---- the square layer in the other configurations bench.py times

def square_inputs():
    cfg = C.SQUARE
    x_h, w_h, gy_h = cfg.x(), cfg.w(), cfg.gy()
    gy_s = W.f32_to_bf16_bits(O.decode(O.BF16, gy_h).astype(np.float32) *
                              np.float32(C.INIT_SCALE)).reshape(gy_h.shape)
    return x_h, w_h, gy_s


def sampled_vec_check(got_dev, out_fmt, A, fa, B, fb, ia, ib, n_pts, seed, what, post=1.0):
    """Sampled outputs against the oracle's vector-scaled GEMM (post scales
    the reference, e.g. by 1/loss scale for unscaled gradients)."""
    M, N = got_dev.shape
    rng = np.random.default_rng(seed)
    ii = np.concatenate([rng.integers(0, M, n_pts), [0, M - 1, 0, M - 1]])
    jj = np.concatenate([rng.integers(0, N, n_pts), [0, N - 1, N - 1, 0]])
    ia = np.broadcast_to(np.asarray(ia, np.float64), (A.shape[0],))
    ib = np.broadcast_to(np.asarray(ib, np.float64), (B.shape[0],))
    c_ref = O.gemm_vec_at(A, fa, B, fb, ia, ib, ii, jj).astype(np.float64) * post
    ad = O.gemm_absdot_vec_at(A, fa, B, fb, ia, ib, ii, jj) * post
    got = host16(got_dev)[ii, jj]
    return check_gemm_values(O.decode(out_fmt, got), c_ref, ad, A.shape[1], out_fmt, what)


def test_square_layer_fused_unscale_step():
    """The step bench.py times: bf16 forward, fp16 backward with the unscale
    and check fused into the GEMM epilogues, update.  Against the oracle
    (codes, scales, sampled unscaled gradients, flag, scaler state) and bit
    for bit against the unfused backward + unscale pass."""
    x_h, w_h, gy_s = square_inputs()
    M, K = x_h.shape
    N = w_h.shape[0]
    x, w, gy = dev16(x_h), dev16(w_h), dev16(gy_s)
    saved = F.LinearSaved(M, N, K)
    ws = F.LinearBwdWs(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
    scale = torch.tensor([C.INIT_SCALE], dtype=torch.float32, device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    log("fused step: GPU")
    F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
    F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
    f_gpu = int(found.item())
    F.amp_update_scale(scale, tracker, found, C.GROWTH, C.BACKOFF, C.INTERVAL)
    torch.cuda.synchronize()
    # the unfused pair on the same saved state
    gx2 = torch.empty_like(gx)
    gw2 = torch.empty_like(gw)
    ws2 = F.LinearBwdWs(M, N)
    found2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    one_scale = torch.tensor([C.INIT_SCALE], dtype=torch.float32, device=DEV)
    F.fp8_scaled_linear_bwd(gy, saved, ws2, gx2, gw2, F.OUT_F16)
    F.amp_unscale_check([gx2, gw2], one_scale, found2)
    torch.cuda.synchronize()
    assert np.array_equal(host16(gx), host16(gx2)) and np.array_equal(host16(gw), host16(gw2))
    assert f_gpu == int(found2.item()) == 0
    log("fused step: oracle")
    xq, wq = O.to_fp8(x_h, O.E4M3FN), O.to_fp8(w_h, O.E4M3FN)
    gq = O.to_fp8(gy_s, O.E5M2)
    for rec, sc, nm in ((saved.x_sc, xq.sc, "x"), (saved.w_sc, wq.sc, "W"), (ws.gy_sc, gq.sc, "gy")):
        check_rec(rec, sc, f"fused {nm}")
    assert_codes_equal(O.E5M2, ws.gy_q.cpu().numpy(), gq.q, "gy_q")
    assert_codes_equal(O.E5M2, ws.gy_qT.cpu().numpy(), gq.qT, "gy_qT")
    inv_s = float(np.float32(1.0) / np.float32(C.INIT_SCALE))
    sampled_vec_check(gx, O.F16, gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv, 2048, 40,
                      "fused dgrad", inv_s)
    sampled_vec_check(gw, O.F16, gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.sc.inv, xq.sc.inv, 2048, 41,
                      "fused wgrad", inv_s)
    st = O.update_scale(O.ScalerState(np.float32(C.INIT_SCALE), 0), 0, C.GROWTH, C.BACKOFF,
                        C.INTERVAL)
    assert float(scale.item()) == float(st.scale) and int(tracker.item()) == st.tracker


def test_square_layer_delayed_steps():
    """bench.py's delayed-scaling step: histories of 16 starting at 1.0, three
    steps on the same tensors; histories, codes and scales bit-exact every
    step, sampled GEMM outputs of the last."""
    x_h, w_h, gy_s = square_inputs()
    M, K = x_h.shape
    N = w_h.shape[0]
    x, w, gy = dev16(x_h), dev16(w_h), dev16(gy_s)
    saved = F.LinearSaved(M, N, K)
    ws = F.LinearBwdWs(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
    hx, hw, hg = (torch.ones(16, dtype=torch.float32, device=DEV) for _ in range(3))
    rhx = rhw = rhg = np.ones(16, np.float32)
    for step in range(3):
        log(f"delayed step {step}")
        F.fp8_scaled_linear_fwd_delayed(x, w, saved, hx, hw, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_delayed(gy, saved, ws, hg, gx, gw, F.OUT_F16)
        torch.cuda.synchronize()
        xq = O.to_fp8_delayed(x_h, O.E4M3FN, rhx)
        wq = O.to_fp8_delayed(w_h, O.E4M3FN, rhw)
        gq = O.to_fp8_delayed(gy_s, O.E5M2, rhg)
        rhx, rhw, rhg = xq.hist, wq.hist, gq.hist
        for got, ref, nm in ((hx, rhx, "hist_x"), (hw, rhw, "hist_w"), (hg, rhg, "hist_gy")):
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (nm, step)
        for rec, sc, nm in ((saved.x_sc, xq.sc, "x"), (saved.w_sc, wq.sc, "W"), (ws.gy_sc, gq.sc, "gy")):
            r = rec.read()
            assert r["scale"] == sc.scale and r["inv"] == sc.inv, (nm, step)
        for got, ref, fmt, nm in ((saved.x_q, xq.q, O.E4M3FN, "x_q"), (saved.w_qT, wq.qT, O.E4M3FN, "w_qT"),
                                  (ws.gy_qT, gq.qT, O.E5M2, "gy_qT")):
            assert_codes_equal(fmt, got.cpu().numpy(), ref, f"{nm} step {step}")
    sampled_gemm_check(y, O.BF16, xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, 1024, 50,
                       "delayed fwd")
    sampled_gemm_check(gx, O.F16, gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv, 1024, 51,
                       "delayed dgrad")
    sampled_gemm_check(gw, O.F16, gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.sc.inv, xq.sc.inv, 1024, 52,
                       "delayed wgrad")


def test_square_layer_rowwise():
    """bench.py's row-wise step: codes and scale vectors of x, W and gy (by
    rows and by columns) bit-exact, sampled GEMM outputs of all three."""
    x_h, w_h, gy_s = square_inputs()
    M, K = x_h.shape
    N = w_h.shape[0]
    saved = F.LinearSavedRW(M, N, K)
    ws = F.LinearBwdWsRW(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
    log("row-wise: GPU")
    F.fp8_scaled_linear_fwd_rowwise(dev16(x_h), dev16(w_h), saved, y, F.OUT_BF16)
    F.fp8_scaled_linear_bwd_rowwise(dev16(gy_s), saved, ws, gx, gw, F.OUT_F16)
    torch.cuda.synchronize()
    log("row-wise: oracle")
    xq, wq = O.to_fp8_rowwise(x_h, O.E4M3FN), O.to_fp8_rowwise(w_h, O.E4M3FN)
    gq = O.to_fp8_rowwise(gy_s, O.E5M2)
    for got, ref, fmt, nm in ((saved.x_q, xq.q, O.E4M3FN, "x_q"), (saved.x_qT, xq.qT, O.E4M3FN, "x_qT"),
                              (saved.w_q, wq.q, O.E4M3FN, "w_q"), (saved.w_qT, wq.qT, O.E4M3FN, "w_qT"),
                              (ws.gy_q, gq.q, O.E5M2, "gy_q"), (ws.gy_qT, gq.qT, O.E5M2, "gy_qT")):
        assert_codes_equal(fmt, got.cpu().numpy(), ref, f"row-wise {nm}")
    for amax, inv, ref, nm in ((saved.x_row_amax, saved.x_row_inv, xq.rows, "x rows"),
                               (saved.x_col_amax, saved.x_col_inv, xq.cols, "x cols"),
                               (saved.w_row_amax, saved.w_row_inv, wq.rows, "w rows"),
                               (saved.w_col_amax, saved.w_col_inv, wq.cols, "w cols"),
                               (ws.gy_row_amax, ws.gy_row_inv, gq.rows, "gy rows"),
                               (ws.gy_col_amax, ws.gy_col_inv, gq.cols, "gy cols")):
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), ref.amax_bits), nm
        assert np.array_equal(inv.cpu().numpy().view(np.uint64), ref.inv.view(np.uint64)), nm
    sampled_vec_check(y, O.BF16, xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.rows.inv, wq.rows.inv, 1024,
                      60, "row-wise fwd")
    sampled_vec_check(gx, O.F16, gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.rows.inv, wq.cols.inv, 1024,
                      61, "row-wise dgrad")
    sampled_vec_check(gw, O.F16, gq.qT, O.E5M2, xq.qT, O.E4M3FN, gq.cols.inv, xq.cols.inv, 1024,
                      62, "row-wise wgrad")
