"""Benchmark of the FP8 per-tensor scaled linear layer + GradScaler step on one
MI355X.

One step = the whole hot path on the square 4096 x 4096 x 4096 layer (bf16
x ~N(0,1) with 0.1% outliers x50, W ~N(0,0.02), gy ~N(0,1e-4), seeded):
  forward:  amax(x), amax(W) -> fp64 scales -> e4m3 codes + transposed copies
            -> y = x W^T (bf16)
  backward: gy carries the loss scale 65536 (fp16 AMP); amax(gy) -> e5m2 codes
            + transposed copy -> dgrad gx = gy W and wgrad gW = gy^T x (fp16)
  scaler:   unscale gx, gW in place + non-finite check -> update()
all through the C ABI on one stream, inputs resident in HBM.

Prints one JSON line.  `value` is the step's GEMM throughput (3 GEMMs,
2 M N K flops each) in TFLOP/s.  The line also carries, each measured with HIP
events on the launch stream: every kernel's average duration with the step's
operands, the roofline of the dominant kernel (the GEMM), the bandwidth of the
memory-bound kernels at HBM scale (a 2^28-element quantize pass and a
200-tensor, ~1.7e9-element unscale pass; logical bytes), and the oracle's CPU
throughput on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-linear fwd+bwd TFLOP/s + quantize/unscale GB/s (% MI355X peak)"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
LOSS_SCALE = 65536.0

# HBM bytes of one 4096^3 GEMM launch (mean over the step's three: forward,
# and dgrad/wgrad with the unscale epilogue) from two rocprofv3 --pmc passes of
# this benchmark (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by
# what the same counter reads for a 1 GiB device-to-device copy
# (bench.py --copy-reference: FETCH_SIZE 524,302 KiB -> x2.0, WRITE_SIZE
# 1,048,576 KiB -> x1.0).  Valid only for the GEMM kernel source they were
# taken on; bench.py reports null for any other.
GEMM_TRAFFIC = {"gemm_src_sha256_16": "168b3f1dc221af4c", "fetch_kib": 49267.5, "write_kib": 32768.0,
                "fetch_factor": 2.0, "write_factor": 1.0}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--reps", type=int, default=50, help="launches per kernel timing loop")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true")
    p.add_argument("--no-hbm", action="store_true", help="skip the HBM-scale bandwidth passes")
    p.add_argument("--no-vendor", action="store_true",
                   help="skip timing the vendor library's FP8 GEMM for comparison")
    p.add_argument("--no-mlp", action="store_true",
                   help="skip the MLP-block timing through the PyTorch layer")
    p.add_argument("--copy-reference", action="store_true",
                   help="only copy 1 GiB device-to-device 5 times (calibrates the HBM byte "
                        "counters against a transfer of known size)")
    p.add_argument("--size", type=int, default=4096, help="M = N = K of the square layer")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, fn, reps):
        """Average time of fn over reps back-to-back calls: one event pair around
        the whole loop on the launch stream, after 3 untimed calls, so per-launch
        dispatch latency is not counted (it is hidden between back-to-back
        kernels, as in the step).  Matches the kernel-trace durations."""
        torch = self.torch
        for _ in range(3):
            fn()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(reps):
            fn()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return {"avg_us": 1e3 * t0.elapsed_time(t1) / reps}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "fp8sg runs on one GPU (no multi-GPU path); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_reference:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes": 1 << 30, "copies": 5}), flush=True)
        return

    import fp8_scaled_gemm_amd as F
    import workloads as W
    from workloads.configs import SQUARE, Linear

    cfg = SQUARE if args.size == 4096 else Linear(
        f"square linear {args.size}^3", args.size, args.size, args.size, 2, 1.0, 0.02, 1e-4,
        1e-3, 50.0)
    M, N, K = cfg.M, cfg.N, cfg.K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    F.lib()

    log(f"generating inputs for {cfg.name}")
    x_h, w_h, gy_h = cfg.x(), cfg.w(), cfg.gy()
    gy_s_h = W.f32_to_bf16_bits(
        (gy_h.view(np.uint16).astype(np.uint32) << 16).view(np.float32) * np.float32(LOSS_SCALE)
    ).reshape(gy_h.shape)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, w, gy = to_dev(x_h), to_dev(w_h), to_dev(gy_s_h)
    saved = F.LinearSaved(M, N, K, device=dev)
    ws = F.LinearBwdWs(M, N, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gx = torch.empty((M, K), dtype=torch.float16, device=dev)
    gw = torch.empty((N, K), dtype=torch.float16, device=dev)
    scale = torch.tensor([LOSS_SCALE], dtype=torch.float32, device=dev)
    tracker = torch.zeros(1, dtype=torch.int32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        # the backward GEMMs write fp16 gx, gW already unscaled and checked
        # (the same bits and flag as an fp16 backward + amp_unscale_check)
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    def step_unfused():
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, F.OUT_F16)
        F.amp_unscale_check([gx, gw], scale, found)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    # the GPU comes out of host-side input generation idle and its clock takes
    # tens of milliseconds to settle: about 0.2 s of steps first, untimed
    log("pre-warm (0.2 s of steps)")
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- the timed region: exactly `steps` steps
    log(f"timing {args.steps} steps")
    # events also every `chunk` steps (recording one does not synchronise):
    # the median and minimum chunk give the spread inside the timed region
    chunk = max(1, args.steps // 10)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range((args.steps + chunk - 1) // chunk + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        if (i + 1) % chunk == 0 or i + 1 == args.steps:
            marks[(i + chunk) // chunk].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t0, t1 = marks[0], marks[-1]
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per_chunk = sorted(marks[k].elapsed_time(marks[k + 1]) / min(chunk, args.steps - k * chunk)
                       for k in range(len(marks) - 1))
    spread = {"chunks": len(per_chunk), "steps_per_chunk": chunk,
              "median_ms_per_step": round(per_chunk[len(per_chunk) // 2], 4),
              "min_ms_per_step": round(per_chunk[0], 4)}
    gemm_flops = 3 * 2.0 * M * N * K
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # ---- the same step with the unscale as its own pass over gx and gW
    for _ in range(args.warmup):
        step_unfused()
    torch.cuda.synchronize()
    u0 = torch.cuda.Event(enable_timing=True)
    u1 = torch.cuda.Event(enable_timing=True)
    u0.record(stream)
    for _ in range(args.steps):
        step_unfused()
    u1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = u0.elapsed_time(u1) / args.steps

    # ---- the same step with delayed scaling of x, W and gy (history of 16)
    hx, hw, hg = (torch.ones(16, dtype=torch.float32, device=dev) for _ in range(3))

    def step_delayed():
        F.fp8_scaled_linear_fwd_delayed(x, w, saved, hx, hw, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_delayed_unscale(gy, saved, ws, hg, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    for _ in range(args.warmup):
        step_delayed()
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        step_delayed()
    d1.record(stream)
    torch.cuda.synchronize()
    ms_delayed = d0.elapsed_time(d1) / args.steps

    # ---- the same step with row-wise scaling (one scale per row of every
    # operand along its non-contraction dimension)
    saved_rw = F.LinearSavedRW(M, N, K, device=dev)
    ws_rw = F.LinearBwdWsRW(M, N, device=dev)
    y_rw, gx_rw, gw_rw = torch.empty_like(y), torch.empty_like(gx), torch.empty_like(gw)

    def step_rowwise():
        F.fp8_scaled_linear_fwd_rowwise(x, w, saved_rw, y_rw, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_rowwise_unscale(gy, saved_rw, ws_rw, scale, found, gx_rw, gw_rw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    for _ in range(args.warmup):
        step_rowwise()
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(args.steps):
        step_rowwise()
    r1.record(stream)
    torch.cuda.synchronize()
    ms_rowwise = r0.elapsed_time(r1) / args.steps

    # ---- per-kernel timings on the same stream, same operands as the step
    log("per-kernel timings")
    T = Timer(torch, stream)
    inv = lambda rec: rec.inv_ptr()
    kern = {}
    kern["gemm_fwd_e4m3xe4m3"] = T.run(lambda: F.fp8_gemm(
        saved.x_q, F.E4M3FN, saved.w_q, F.E4M3FN, inv(saved.x_sc), inv(saved.w_sc), y,
        F.OUT_BF16), args.reps)
    # dgrad and wgrad as the step runs them: fp16 out, unscaled and checked in the epilogue
    fz0 = torch.zeros(1, dtype=torch.int32, device=dev)
    kern["gemm_dgrad_e5m2xe4m3"] = T.run(lambda: F.fp8_gemm_unscale(
        ws.gy_q, F.E5M2, saved.w_qT, F.E4M3FN, inv(ws.gy_sc), inv(saved.w_sc), scale, fz0,
        gx), args.reps)
    kern["gemm_wgrad_e5m2xe4m3"] = T.run(lambda: F.fp8_gemm_unscale(
        ws.gy_qT, F.E5M2, saved.x_qT, F.E4M3FN, inv(ws.gy_sc), inv(saved.x_sc), scale, fz0,
        gw), args.reps)
    kern["gemm_dgrad_plain_f16"] = T.run(lambda: F.fp8_gemm(
        ws.gy_q, F.E5M2, saved.w_qT, F.E4M3FN, inv(ws.gy_sc), inv(saved.w_sc), gx,
        F.OUT_F16), args.reps)
    rec = F.ScaleRec(device=dev)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    qT = torch.empty((K, M), dtype=torch.uint8, device=dev)
    kern["amax_x_standalone"] = T.run(lambda: F.fp8_amax(x, rec), args.reps)
    kern["quantize_transpose_x"] = T.run(lambda: F.fp8_quantize(x, F.E4M3FN, rec, q, qT),
                                         args.reps)
    g16 = [torch.empty_like(gx).copy_(gx), torch.empty_like(gw).copy_(gw)]
    one = torch.ones(1, dtype=torch.float32, device=dev)
    fz = torch.zeros(1, dtype=torch.int32, device=dev)
    kern["unscale_check_gx_gw"] = T.run(lambda: F.amp_unscale_check(g16, one, fz), args.reps)
    # the whole backward (gy cast + both GEMMs), fp16 out, without and with the fused unscale
    kern["linear_bwd_f16"] = T.run(lambda: F.fp8_scaled_linear_bwd(gy, saved, ws, g16[0], g16[1],
                                                                   F.OUT_F16), args.reps)
    kern["linear_bwd_unscale"] = T.run(lambda: F.fp8_scaled_linear_bwd_unscale(
        gy, saved, ws, scale, fz, g16[0], g16[1]), args.reps)
    kern["update_scale"] = T.run(lambda: F.amp_update_scale(scale, tracker, found, 2.0, 0.5,
                                                            2000), args.reps)
    rs, cs = F.RowScalesDev(M, device=dev), F.RowScalesDev(K, device=dev)
    kern["quantize_rowwise_transpose_x"] = T.run(
        lambda: F.fp8_quantize_rowwise(x, F.E4M3FN, rs, q, cs, qT), args.reps)
    kern["gemm_rowwise_fwd_e4m3xe4m3"] = T.run(lambda: F.fp8_gemm_rowwise(
        saved_rw.x_q, F.E4M3FN, saved_rw.w_q, F.E4M3FN, saved_rw.x_row_inv, saved_rw.w_row_inv,
        y_rw, F.OUT_BF16), args.reps)
    del g16, q, qT, rs, cs

    # ---- the vendor library's FP8 GEMM (hipBLASLt through torch._scaled_mm) on
    # the forward's codes and inverse scales: context for the GEMM's roofline
    # fraction, timed the same way; not part of the step
    vendor = None
    if not args.no_vendor:
        try:
            a8 = saved.x_q.view(torch.float8_e4m3fn)
            b8 = saved.w_q.view(torch.float8_e4m3fn).t()  # [K, N], column-major
            sa = torch.tensor([saved.x_sc.read()["inv32"]], dtype=torch.float32, device=dev)
            sb = torch.tensor([saved.w_sc.read()["inv32"]], dtype=torch.float32, device=dev)
            mm = lambda: torch._scaled_mm(a8, b8, scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
            v_us = T.run(mm, args.reps)["avg_us"]
            ref = mm().float()
            ours = y.float()
            vendor = {"library": "hipBLASLt via torch._scaled_mm (e4m3fn x e4m3fn -> bf16)",
                      "gemm_us": round(v_us, 2),
                      "TFLOPs": round(2.0 * M * N * K / (v_us * 1e-6) / 1e12, 1),
                      "ours_fwd_gemm_us": round(kern["gemm_fwd_e4m3xe4m3"]["avg_us"], 2),
                      "speedup_ours_over_vendor": round(
                          v_us / kern["gemm_fwd_e4m3xe4m3"]["avg_us"], 3),
                      "max_abs_diff_over_max_abs": float((ref - ours).abs().max() /
                                                         ours.abs().max())}
        except Exception as e:  # an unsupported layout or dtype on this torch build
            vendor = {"error": f"{type(e).__name__}: {e}"[:200]}

    gemm_avg_us = sum(kern[k]["avg_us"] for k in ("gemm_fwd_e4m3xe4m3", "gemm_dgrad_e5m2xe4m3",
                                                  "gemm_wgrad_e5m2xe4m3")) / 3
    gemm_tflops = 2.0 * M * N * K / (gemm_avg_us * 1e-6) / 1e12
    traffic = None
    import hashlib
    src = os.path.join(ROOT, "fp8_scaled_gemm_amd", "csrc", "gemm_kernels.hpp")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if (M, N, K) == (4096, 4096, 4096) and digest == GEMM_TRAFFIC["gemm_src_sha256_16"]:
        traffic = 1024.0 * (GEMM_TRAFFIC["fetch_kib"] * GEMM_TRAFFIC["fetch_factor"] +
                            GEMM_TRAFFIC["write_kib"] * GEMM_TRAFFIC["write_factor"])

    # ---- memory-bound kernels at HBM scale (working sets far above the 256 MB
    # Infinity Cache): amax + e4m3 quantize of a 2^28-element bf16 tensor
    # (magnitudes 10^U(-6,3)), and unscale + check over 200 fp16 gradients of
    # log-uniform sizes 4K..64M
    hbm = {}
    if not args.no_hbm:
        from workloads import configs as C
        log("HBM-scale quantize pass")
        big = torch.from_numpy(C.quant_act().view(np.int16)).view(torch.bfloat16).to(dev)
        bq = torch.empty(big.shape, dtype=torch.uint8, device=dev)
        brec = F.ScaleRec(device=dev)
        r_amax = T.run(lambda: F.fp8_amax(big, brec), 10)
        r_quant = T.run(lambda: F.fp8_quantize(big, F.E4M3FN, brec, bq), 10)
        nb = big.numel()
        hbm["amax_GBps"] = 2.0 * nb / (r_amax["avg_us"] * 1e-6) / 1e9
        hbm["quantize_GBps"] = 3.0 * nb / (r_quant["avg_us"] * 1e-6) / 1e9
        hbm["amax_plus_quantize_GBps"] = 5.0 * nb / ((r_amax["avg_us"] + r_quant["avg_us"]) * 1e-6) / 1e9
        kern["amax_2p28"] = r_amax
        kern["quantize_2p28"] = r_quant
        # delayed scaling: one pass (scale from the history, current amax reduced
        # on the way): 2 B read + 1 B written per element
        amax_big = float(np.array([brec.read()["amax_bits"]], np.uint32).view(np.float32)[0])
        bh = torch.full((16,), amax_big, dtype=torch.float32, device=dev)
        r_del = T.run(lambda: F.fp8_quantize_delayed(big, F.E4M3FN, brec, bh, bq), 10)
        hbm["quantize_delayed_GBps"] = 3.0 * nb / (r_del["avg_us"] * 1e-6) / 1e9
        kern["quantize_delayed_2p28"] = r_del
        # row-wise: amax pass (2 B/elem) + cast with the transposed copy
        # (2 B read + 2 B written), the tensor as a 16384 x 16384 matrix
        side = 1 << 14
        big2 = big.view(side, side)
        bqT = torch.empty((side, side), dtype=torch.uint8, device=dev)
        brs, bcs = F.RowScalesDev(side, device=dev), F.RowScalesDev(side, device=dev)
        r_rw = T.run(lambda: F.fp8_quantize_rowwise(big2, F.E4M3FN, brs, bq.view(side, side), bcs,
                                                     bqT), 10)
        hbm["quantize_rowwise_transpose_GBps"] = 6.0 * nb / (r_rw["avg_us"] * 1e-6) / 1e9
        kern["quantize_rowwise_transpose_2p28"] = r_rw
        del big, bq, bh, big2, bqT
        # the gradient half of the quantize-path workload: an equal-size tensor
        # (magnitudes 10^U(-8,-2)) cast to e5m2
        gbig = torch.from_numpy(C.quant_grad().view(np.int16)).view(torch.bfloat16).to(dev)
        gq = torch.empty(gbig.shape, dtype=torch.uint8, device=dev)
        grec = F.ScaleRec(device=dev)
        r_gamax = T.run(lambda: F.fp8_amax(gbig, grec), 10)
        r_gquant = T.run(lambda: F.fp8_quantize(gbig, F.E5M2, grec, gq), 10)
        hbm["amax_plus_quantize_e5m2_GBps"] = 5.0 * nb / ((r_gamax["avg_us"] + r_gquant["avg_us"]) * 1e-6) / 1e9
        kern["amax_2p28_grad"] = r_gamax
        kern["quantize_e5m2_2p28"] = r_gquant
        del gbig, gq
        log("HBM-scale unscale pass")
        sizes = C.scaler_sizes()
        grads = [(torch.randn(int(n), device=dev) * 0.5).half() for n in sizes]
        r_un = T.run(lambda: F.amp_unscale_check(grads, one, fz), 10)
        ng = int(sizes.sum())
        hbm["unscale_GBps"] = 4.0 * ng / (r_un["avg_us"] * 1e-6) / 1e9
        hbm["unscale_elements"] = ng
        kern["unscale_check_200_tensors"] = r_un
        # the same pass with the global gradient norm (sum of squares) fused in
        nws = torch.empty(F.amp_norm_workspace_len([g.numel() for g in grads]),
                          dtype=torch.float32, device=dev)
        nout = torch.empty(2, dtype=torch.float32, device=dev)
        r_nrm = T.run(lambda: F.amp_unscale_check_norm(grads, one, fz, nws, nout), 10)
        hbm["unscale_norm_GBps"] = 4.0 * ng / (r_nrm["avg_us"] * 1e-6) / 1e9
        kern["unscale_check_norm_200_tensors"] = r_nrm
        del grads, nws
        torch.cuda.empty_cache()

    small = small_layer(torch, F, dev, stream, T)

    mlp = None
    if not args.no_mlp:
        log("MLP block through the PyTorch layer")
        mlp = mlp_block(torch, F, dev, stream)
        torch.cuda.empty_cache()

    # ---- sampled check of the step's outputs against the oracle
    check = None
    if not args.no_check:
        log("sampled oracle check")
        step()  # the delayed-scaling step shares these buffers: restore the dynamic step's
        torch.cuda.synchronize()
        check = sampled_check(np, torch, F, x_h, w_h, gy_s_h, saved, ws, y, M, N, K)
        check["rowwise"] = sampled_check_rowwise(np, torch, x_h, w_h, saved_rw, y_rw, M, N, K)

    # ---- oracle on the host cores, bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        log("oracle CPU baseline")
        cpu = cpu_baseline(np, saved, M, N, K)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: FP8 linear fwd+dgrad+wgrad with fused transposed "
                               "copies + GradScaler unscale/check (fused into the dgrad/wgrad "
                               "epilogues) and update",
                   "M": M, "N": N, "K": K, "x": "bf16 N(0,1), 0.1% outliers x50",
                   "W": "bf16 N(0,0.02)", "gy": "bf16 N(0,1e-4) x loss scale 65536",
                   "y": "bf16", "grads": "fp16", "formats": "e4m3fn x/W, e5m2 gy"},
        "step_pct_of_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "step_spread": spread,
        "step_unfused_unscale": {"ms_per_step": round(ms_unfused, 4),
                                 "TFLOPs": round(gemm_flops / (ms_unfused * 1e-3) / 1e12, 2)},
        "step_delayed_scaling": {"ms_per_step": round(ms_delayed, 4),
                                 "TFLOPs": round(gemm_flops / (ms_delayed * 1e-3) / 1e12, 2),
                                 "history": 16},
        "step_rowwise_scaling": {"ms_per_step": round(ms_rowwise, 4),
                                 "TFLOPs": round(gemm_flops / (ms_rowwise * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM, counter-measured)",
                     "kernel": "k_gemm_pingpong (3 GEMMs of the step, 2*M*N*K flops per launch)"},
        "vendor_gemm": vendor,
        "hbm_scale": {k: (round(v, 1) if isinstance(v, float) else v) for k, v in hbm.items()},
        "hbm_frac": {k[:-5]: round(v / PEAK_HBM_GBPS, 4) for k, v in hbm.items()
                     if k.endswith("_GBps")},
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "wall_s_timed_region": round(wall, 4),
        "check": check,
        "small_layer": small,
        "mlp_block": mlp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def small_layer(torch, F, dev, stream, T, reps=200):
    """The small layer (B=64, K=128, N=256): launch-latency bound, so its
    time per phase and its kernel launches are reported, eager and replayed
    from a HIP graph."""
    from workloads.configs import SMALL as S
    import numpy as np
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    x, w, gy = to_dev(S.x()), to_dev(S.w()), to_dev(S.gy())
    saved = F.LinearSaved(S.M, S.N, S.K, device=dev)
    ws = F.LinearBwdWs(S.M, S.N, device=dev)
    y = torch.empty((S.M, S.N), dtype=torch.bfloat16, device=dev)
    gx = torch.empty((S.M, S.K), dtype=torch.float16, device=dev)
    gw = torch.empty((S.N, S.K), dtype=torch.float16, device=dev)
    scale = torch.tensor([65536.0], dtype=torch.float32, device=dev)
    tracker = torch.zeros(1, dtype=torch.int32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)
    fwd = lambda: F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
    bwd = lambda: F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, F.OUT_F16)
    scaler = lambda: (F.amp_unscale_check([gx, gw], scale, found),
                      F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000))

    def step():
        fwd()
        bwd()
        scaler()

    def step_fused():  # unscale + check in the backward epilogues: update only after it
        fwd()
        F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    def replay_us(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            fn()
        return round(T.run(g.replay, reps)["avg_us"], 2)

    out = {"workload": "small linear B=64 K=128 N=256 + GradScaler step (init 65536, "
                       "interval 2000)",
           "fwd_us": round(T.run(fwd, reps)["avg_us"], 2),
           "bwd_us": round(T.run(bwd, reps)["avg_us"], 2),
           "scaler_step_us": round(T.run(scaler, reps)["avg_us"], 2),
           "step_us": round(T.run(step, reps)["avg_us"], 2),
           "step_fused_unscale_us": round(T.run(step_fused, reps)["avg_us"], 2),
           # tensors of at most 64 Ki elements are cast by one block each with
           # their own amax, and the two backward GEMMs share a launch
           "launches": {"fwd": 2, "bwd": 2, "scaler_step": 2, "step_fused_unscale": 5}}
    out["step_graph_replay_us"] = replay_us(step)
    out["step_fused_unscale_graph_replay_us"] = replay_us(step_fused)
    out["TFLOPs_eager"] = round(3 * 2.0 * S.M * S.N * S.K / (out["step_us"] * 1e-6) / 1e12, 4)
    return out


def mlp_block(torch, F, dev, stream, steps=10, warmup=3):
    """The transformer MLP block's three FP8 linears (gate, up: 4096 -> 14336;
    down: 14336 -> 4096; 8192 tokens) trained through Float8Linear and autograd
    (x shared by gate and up, as in the block; each module casts its own input),
    against the same nine GEMMs driven directly through the C-ABI, where x is
    reduced and cast once for gate and up.  Synthetic device data at the
    workload's shapes and standard deviations."""
    import fp8_scaled_gemm_amd.nn as FN
    T, H, Fd = 8192, 4096, 14336
    bf = dict(dtype=torch.bfloat16, device=dev)
    shapes = {"gate": (H, Fd), "up": (H, Fd), "down": (Fd, H)}
    mods = {n: FN.Float8Linear(k, o, device=dev) for n, (k, o) in shapes.items()}
    for m in mods.values():
        with torch.no_grad():
            m.weight.normal_(0.0, 0.02)
    x = torch.randn(T, H, **bf).requires_grad_(True)
    h = torch.randn(T, Fd, **bf).requires_grad_(True)
    gys = {"gate": torch.randn(T, Fd, **bf) * 1e-4, "up": torch.randn(T, Fd, **bf) * 1e-4,
           "down": torch.randn(T, H, **bf) * 1e-4}

    def autograd_step():
        for t in [x, h] + [m.weight for m in mods.values()]:
            t.grad = None
        outs = [mods["gate"](x), mods["up"](x), mods["down"](h)]
        torch.autograd.backward(outs, [gys["gate"], gys["up"], gys["down"]])

    direct = {}
    for n, (k, o) in shapes.items():
        inp = x if n != "down" else h
        direct[n] = dict(inp=inp.detach(), w=mods[n].weight.detach(),
                         saved=F.LinearSaved(T, o, k, device=dev), ws=F.LinearBwdWs(T, o, device=dev),
                         y=torch.empty(T, o, **bf), gx=torch.empty(T, k, **bf),
                         gw=torch.empty(o, k, **bf))
    # up shares gate's input: its saved x codes, transposed codes and scale
    # record are gate's, so x is reduced and cast once per step
    g_sv, u = direct["gate"]["saved"], direct["up"]
    u["saved"] = F.LinearSaved(T, Fd, H, tensors=(g_sv.x_q, g_sv.x_qT, u["saved"].w_q,
                                                  u["saved"].w_qT, u["saved"].recs))
    u["saved"].x_sc = g_sv.x_sc

    def direct_step():
        for n, d in direct.items():
            if n == "up":  # W_up alone: amax, cast (+ transposed copy), GEMM on gate's x codes
                sv = d["saved"]
                F.fp8_amax(d["w"], sv.w_sc)
                F.fp8_quantize(d["w"], F.E4M3FN, sv.w_sc, sv.w_q, sv.w_qT)
                F.fp8_gemm(sv.x_q, F.E4M3FN, sv.w_q, F.E4M3FN, sv.x_sc.inv_ptr(), sv.w_sc.inv_ptr(),
                           d["y"], F.OUT_BF16)
            else:
                F.fp8_scaled_linear_fwd(d["inp"], d["w"], d["saved"], d["y"], F.OUT_BF16)
        for n, d in direct.items():
            F.fp8_scaled_linear_bwd(gys[n], d["saved"], d["ws"], d["gx"], d["gw"], F.OUT_BF16)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_auto, ms_direct = timed(autograd_step), timed(direct_step)
    flops = 9 * 2.0 * T * Fd * H
    return {"workload": "MLP block T=8192 H=4096 F=14336: gate/up/down fwd+dgrad+wgrad",
            "autograd_ms_per_step": round(ms_auto, 4),
            "autograd_TFLOPs": round(flops / (ms_auto * 1e-3) / 1e12, 1),
            "direct_abi_ms_per_step": round(ms_direct, 4),
            "direct_abi_TFLOPs": round(flops / (ms_direct * 1e-3) / 1e12, 1)}


def sampled_check(np, torch, F, x_h, w_h, gy_h, saved, ws, y, M, N, K, n_pts=256):
    """Recompute codes and scales with the oracle from the same host inputs and
    compare them with the step's device buffers; check sampled GEMM outputs."""
    import oracle as O
    from tests.parity import assert_codes_equal, check_gemm_values
    xq = O.to_fp8(x_h, O.E4M3FN)
    wq = O.to_fp8(w_h, O.E4M3FN)
    gq = O.to_fp8(gy_h, O.E5M2)
    for got, ref, fmt in ((saved.x_q, xq.q, O.E4M3FN), (saved.w_qT, wq.qT, O.E4M3FN),
                          (ws.gy_qT, gq.qT, O.E5M2)):
        assert_codes_equal(fmt, got.cpu().numpy(), ref)
    for rec, sc in ((saved.x_sc, xq.sc), (saved.w_sc, wq.sc), (ws.gy_sc, gq.sc)):
        r = rec.read()
        assert r["amax_bits"] == sc.amax_bits and r["inv"] == sc.inv
    rng = np.random.default_rng(0)
    ii = rng.integers(0, M, n_pts)
    jj = rng.integers(0, N, n_pts)
    c_ref = O.gemm_at(xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, ii, jj)
    ad = O.gemm_absdot_at(xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.sc.inv, wq.sc.inv, ii, jj)
    y_h = y.view(torch.int16).cpu().numpy().view(np.uint16)[ii, jj]
    nw = check_gemm_values(O.decode(O.BF16, y_h), c_ref, ad, K, O.BF16, "bench y")
    return {"codes_and_scales": "bit-exact", "gemm_fwd_samples": n_pts, "ok": True,
            "max_abs_err_over_max_abs": float(nw)}


def sampled_check_rowwise(np, torch, x_h, w_h, saved, y, M, N, K, n_pts=256):
    """The row-wise step's forward: codes and scale vectors of x and W against
    the oracle's row-wise cast, sampled outputs of y."""
    import oracle as O
    from tests.parity import assert_codes_equal, check_gemm_values
    xq = O.to_fp8_rowwise(x_h, O.E4M3FN)
    wq = O.to_fp8_rowwise(w_h, O.E4M3FN)
    for got, ref in ((saved.x_q, xq.q), (saved.x_qT, xq.qT), (saved.w_q, wq.q),
                     (saved.w_qT, wq.qT)):
        assert_codes_equal(O.E4M3FN, got.cpu().numpy(), ref)
    for got, ref in ((saved.x_row_inv, xq.rows.inv), (saved.x_col_inv, xq.cols.inv),
                     (saved.w_row_inv, wq.rows.inv), (saved.w_col_inv, wq.cols.inv)):
        assert np.array_equal(got.cpu().numpy().view(np.uint64), ref.view(np.uint64))
    rng = np.random.default_rng(1)
    ii = rng.integers(0, M, n_pts)
    jj = rng.integers(0, N, n_pts)
    c_ref = O.gemm_vec_at(xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.rows.inv, wq.rows.inv, ii, jj)
    ad = O.gemm_absdot_vec_at(xq.q, O.E4M3FN, wq.q, O.E4M3FN, xq.rows.inv, wq.rows.inv, ii, jj)
    y_h = y.view(torch.int16).cpu().numpy().view(np.uint16)[ii, jj]
    nw = check_gemm_values(O.decode(O.BF16, y_h), c_ref, ad, K, O.BF16, "bench y rowwise")
    return {"codes_and_scale_vectors": "bit-exact", "gemm_fwd_samples": n_pts, "ok": True,
            "max_abs_err_over_max_abs": float(nw)}


def cpu_baseline(np, saved, M, N, K, rows=None):
    """The oracle (plain C, OpenMP) on the host cores: the forward GEMM on a
    slab of rows, on the step's own FP8 codes.  Throughput in the metric's
    unit (TFLOP/s)."""
    import oracle as O
    A = saved.x_q.cpu().numpy()
    B = saved.w_q.cpu().numpy()
    threads = O.num_threads()
    if rows is None:  # size the slab for about 10 s of wall time on these cores
        probe = max(1, threads)
        t = time.perf_counter()
        O.gemm(A[:probe], O.E4M3FN, B, O.E4M3FN, 1.0, 1.0)
        per_row = (time.perf_counter() - t) / probe
        rows = int(min(M, max(probe, 10.0 / max(per_row, 1e-9))))
        rows = max(threads, rows - rows % max(threads, 1))
    t = time.perf_counter()
    O.gemm(A[:rows], O.E4M3FN, B, O.E4M3FN, 1.0, 1.0)
    dt = time.perf_counter() - t
    flops = 2.0 * rows * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"forward GEMM on {rows} of {M} rows ({rows}x{N}x{K}, fp32 sequential "
                      f"accumulation), {dt:.2f} s wall"}


if __name__ == "__main__":
    main()
