"""Benchmark of the FP8 per-tensor scaled linear layers + GradScaler step on one
MI355X.

One step = the whole hot path on the transformer MLP block (tokens T=8192,
hidden H=4096, ffn F=14336; gate and up W [14336,4096], down W [4096,14336];
bf16 activations x, h ~N(0,1), weights ~N(0,0.02), gradients ~N(0,1e-4), all
seeded; fp16 AMP with loss scale 65536):
  forward:  amax -> fp64 scale -> e4m3 codes of x (once, shared by gate and
            up), h and the three weights -> y = x W^T (bf16) for gate, up, down
  backward: each linear's gradient (carrying the loss scale) amax -> e5m2
            codes -> dgrad gx = gy W and wgrad gW = gy^T x in fp16, the GEMMs
            reading W, x, gy of down contraction-major and gy of gate and
            up, h through the transposed copies their casts write (--layout
            chooses other mixes), unscaled and checked for inf/NaN in the
            GEMM epilogues
  scaler:   update() of the loss scale on the device
all through the C ABI on one stream, inputs resident in HBM.

Prints one JSON line.  `value` is the step's GEMM throughput (9 GEMMs,
2 M N K flops each) in TFLOP/s over the whole step's time.  The line also
carries, each measured with HIP events on the launch stream: every GEMM's and
every cast's average duration with the step's own operands, the roofline of the
dominant kernel (the GEMM), the bandwidth of the memory-bound kernels at HBM
scale (the 2^28-element quantize workload, the 200-tensor GradScaler workload,
16384 x 16384 casts with transposed copies), the square 4096^3 layer and the
small layer as side lines, a sampled oracle check of the step's outputs, and
the oracle's CPU throughput on a slab of the same step.
"""
import argparse
import hashlib
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
GEMM_SRC = os.path.join(ROOT, "fp8_scaled_gemm_amd", "csrc", "gemm_kernels.hpp")

# HBM bytes per GEMM launch of the MLP step (mean over its nine GEMMs) from two
# rocprofv3 --pmc passes of this benchmark (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch), each scaled by what the same counter reads for a 1 GiB
# device-to-device copy (bench.py --copy-reference: FETCH_SIZE x2.0,
# WRITE_SIZE x1.0).  Valid only for the GEMM kernel source they were taken on
# (its hash); bench.py reports null for any other.
GEMM_TRAFFIC = {"gemm_src_sha256_16": "3cb9b645dee0b52f", "fetch_kib": 355144.4,
                "write_kib": 137377.3, "fetch_factor": 2.0, "write_factor": 1.0}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--reps", type=int, default=20, help="launches per kernel timing loop")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true")
    p.add_argument("--no-hbm", action="store_true", help="skip the HBM-scale bandwidth passes")
    p.add_argument("--no-side", action="store_true",
                   help="skip the square-layer, small-layer and autograd side lines")
    p.add_argument("--hbm-only", action="store_true",
                   help="only the HBM-scale passes (for counter runs); prints their figures")
    p.add_argument("--square-only", action="store_true",
                   help="only the square 4096^3 layer's side line (for counter runs)")
    p.add_argument("--layout", choices=("auto", "none", "all"), default="auto",
                   help="which transposed code copies the MLP step's casts write: 'auto' "
                        "(default) those fp8_linear_copies picks (the weight-gradient GEMMs' "
                        "first operand: gy of gate and up, h of down), the other operands read "
                        "contraction-major; 'none': every backward operand read "
                        "contraction-major; 'all': every copy written and read row-major")
    p.add_argument("--copy-reference", action="store_true",
                   help="only copy 1 GiB device-to-device 5 times (calibrates the HBM byte "
                        "counters against a transfer of known size)")
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
        return 1e3 * t0.elapsed_time(t1) / reps


def timed_steps(torch, stream, step, steps, warmup):
    """The timed region: `warmup` untimed steps after about 0.2 s of pre-warm
    steps (the clock settles after host-side input generation), then exactly
    `steps` steps between two events, with an event every steps/10 steps
    (recording one does not synchronise) for the spread."""
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    chunk = max(1, steps // 10)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range((steps + chunk - 1) // chunk + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(steps):
        step()
        if (i + 1) % chunk == 0 or i + 1 == steps:
            marks[(i + chunk) // chunk].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = marks[0].elapsed_time(marks[-1]) / steps
    per_chunk = sorted(marks[k].elapsed_time(marks[k + 1]) / min(chunk, steps - k * chunk)
                       for k in range(len(marks) - 1))
    spread = {"chunks": len(per_chunk), "steps_per_chunk": chunk,
              "median_ms_per_step": round(per_chunk[len(per_chunk) // 2], 4),
              "min_ms_per_step": round(per_chunk[0], 4)}
    return ms, wall, spread


def bf16_dev(torch, np, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def loss_scaled(np, bits):
    """bf16(S * g) for the power-of-two loss scale S: exact, so the FP8 codes of
    the gradient are unchanged and its inverse scale carries S."""
    import workloads as W
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(LOSS_SCALE)
    return W.f32_to_bf16_bits(f).reshape(bits.shape)


# ---------------------------------------------------------------- MLP block

class MlpStep:
    """The MLP block's three FP8 linears with the step's device buffers.

    x is reduced and cast once for gate and up (the same tensor gives the same
    amax and codes): up's forward casts only W_up and runs its GEMM on gate's x
    codes, and up's backward reads gate's saved x codes and scale record."""

    NAMES = ("gate", "up", "down")

    # which tensors' casts write a transposed copy: "auto" asks the library
    # (fp8_linear_copies: the weight gradient's first GEMM operand, read twice
    # as often from LDS as the second, keeps its copy -- gy of gate and up, h
    # for down, whose weight gradient runs with the operands' roles swapped)
    ALL = {"x", "h", "w_gate", "w_up", "w_down", "gy_gate", "gy_up", "gy_down"}

    def __init__(self, np, torch, F, dev, layout="auto", inputs=None):
        from workloads.configs import mlp_linear, MLP_T, MLP_H, MLP_F
        self.F, self.torch, self.layout = F, torch, layout
        self.lin = {n: mlp_linear(n) for n in self.NAMES}
        if layout == "auto":
            self.tr = set()
            for n, L in self.lin.items():
                xt, wt, gt = F.fp8_linear_copies(L.M, L.N, L.K)
                for key, on in ((("h" if n == "down" else "x"), xt), ("w_" + n, wt), ("gy_" + n, gt)):
                    if on:
                        self.tr.add(key)
        else:
            self.tr = set() if layout == "none" else set(self.ALL)
        self.T, self.H, self.Fd = MLP_T, MLP_H, MLP_F
        if inputs is not None:  # (host arrays, device tensors) of another MlpStep
            self.host, self.dev = inputs
        else:
            log("generating the MLP block's inputs")
            self.host = {}
            g = self.lin["gate"]
            self.host["x"] = g.x()
            self.host["h"] = self.lin["down"].x()
            for n in self.NAMES:
                self.host["w_" + n] = self.lin[n].w()
                self.host["gy_" + n] = loss_scaled(np, self.lin[n].gy())
            self.dev = {k: bf16_dev(torch, np, v, dev) for k, v in self.host.items()}
        bf = dict(dtype=torch.bfloat16, device=dev)
        f16 = dict(dtype=torch.float16, device=dev)
        self.saved, self.ws, self.y, self.gx, self.gw = {}, {}, {}, {}, {}
        for n in self.NAMES:
            L = self.lin[n]
            self.saved[n] = F.LinearSaved(L.M, L.N, L.K, device=dev,
                                          x_transposed=("h" if n == "down" else "x") in self.tr,
                                          w_transposed="w_" + n in self.tr)
            self.ws[n] = F.LinearBwdWs(L.M, L.N, device=dev, transposed="gy_" + n in self.tr)
            self.y[n] = torch.empty((L.M, L.N), **bf)
            self.gx[n] = torch.empty((L.M, L.K), **f16)
            self.gw[n] = torch.empty((L.N, L.K), **f16)
        gs, us = self.saved["gate"], self.saved["up"]
        self.saved["up"] = F.LinearSaved(self.T, self.Fd, self.H,
                                         tensors=(gs.x_q, gs.x_qT, us.w_q, us.w_qT, us.recs))
        self.saved["up"].x_sc = gs.x_sc
        self.scale = torch.tensor([LOSS_SCALE], dtype=torch.float32, device=dev)
        self.tracker = torch.zeros(1, dtype=torch.int32, device=dev)
        self.found = torch.zeros(1, dtype=torch.int32, device=dev)

    def inputs(self, n):
        return self.dev["h"] if n == "down" else self.dev["x"]

    def forward(self):
        F, d, sv = self.F, self.dev, self.saved
        F.fp8_scaled_linear_fwd(d["x"], d["w_gate"], sv["gate"], self.y["gate"], F.OUT_BF16)
        u = sv["up"]
        F.fp8_amax(d["w_up"], u.w_sc)
        F.fp8_quantize(d["w_up"], F.E4M3FN, u.w_sc, u.w_q, u.w_qT)
        F.fp8_gemm(u.x_q, F.E4M3FN, u.w_q, F.E4M3FN, u.x_sc.inv_ptr(), u.w_sc.inv_ptr(),
                   self.y["up"], F.OUT_BF16)
        F.fp8_scaled_linear_fwd(d["h"], d["w_down"], sv["down"], self.y["down"], F.OUT_BF16)

    def backward(self):
        F = self.F
        for n in self.NAMES:
            F.fp8_scaled_linear_bwd_unscale(self.dev["gy_" + n], self.saved[n], self.ws[n],
                                            self.scale, self.found, self.gx[n], self.gw[n])

    def step(self):
        self.forward()
        self.backward()
        self.F.amp_update_scale(self.scale, self.tracker, self.found, 2.0, 0.5, 2000)

    def gemms(self):
        """The step's nine GEMMs as (name, flops, call) on the step's operands:
        forward in bf16, dgrad and wgrad with the unscale epilogue."""
        F, out = self.F, []
        fz = self.torch.zeros(1, dtype=self.torch.int32, device=self.scale.device)
        for n in self.NAMES:
            L, sv, ws = self.lin[n], self.saved[n], self.ws[n]
            fl = 2.0 * L.M * L.N * L.K
            out.append((f"{n}_fwd {L.M}x{L.N}x{L.K}", fl, lambda sv=sv, n=n: F.fp8_gemm(
                sv.x_q, F.E4M3FN, sv.w_q, F.E4M3FN, sv.x_sc.inv_ptr(), sv.w_sc.inv_ptr(),
                self.y[n], F.OUT_BF16)))
            # as the layer's backward: a transposed copy where the cast wrote
            # one, else the row-major codes read contraction-major (W as B^T
            # for dgrad; gy as A^T and x as B^T for wgrad)
            wk, gk, xk = sv.w_qT is None, ws.gy_qT is None, sv.x_qT is None
            dg = lambda sv=sv, ws=ws, n=n, wk=wk: F.fp8_gemm_kmajor_unscale(
                ws.gy_q, F.E5M2, 0, sv.w_q if wk else sv.w_qT, F.E4M3FN, wk, ws.gy_sc.inv_ptr(),
                sv.w_sc.inv_ptr(), self.scale, fz, self.gx[n])
            wg = lambda sv=sv, ws=ws, n=n, gk=gk, xk=xk: F.fp8_gemm_kmajor_unscale(
                ws.gy_q if gk else ws.gy_qT, F.E5M2, gk, sv.x_q if xk else sv.x_qT, F.E4M3FN, xk,
                ws.gy_sc.inv_ptr(), sv.x_sc.inv_ptr(), self.scale, fz, self.gw[n])
            out.append((f"{n}_dgrad {L.M}x{L.K}x{L.N}", fl, dg))
            out.append((f"{n}_wgrad {L.N}x{L.K}x{L.M}", fl, wg))
        return out

    def casts(self):
        """The step's eight casts (amax, then quantize, with the transposed copy
        where the step keeps one) as (name, elements, bytes, call), on fresh
        records of their own."""
        F, out = self.F, []
        d = self.dev
        for name, t, fmt in (("x", d["x"], F.E4M3FN), ("h", d["h"], F.E4M3FN),
                             ("w_gate", d["w_gate"], F.E4M3FN), ("w_up", d["w_up"], F.E4M3FN),
                             ("w_down", d["w_down"], F.E4M3FN), ("gy_gate", d["gy_gate"], F.E5M2),
                             ("gy_up", d["gy_up"], F.E5M2), ("gy_down", d["gy_down"], F.E5M2)):
            rec = F.ScaleRec(device=t.device)
            q = self.torch.empty(t.shape, dtype=self.torch.uint8, device=t.device)
            qT = (self.torch.empty((t.shape[1], t.shape[0]), dtype=self.torch.uint8, device=t.device)
                  if name in self.tr else None)

            def call(t=t, fmt=fmt, rec=rec, q=q, qT=qT):
                F.fp8_amax(t, rec)
                F.fp8_quantize(t, fmt, rec, q, qT)
            # amax reads 2 B; the cast reads 2 B and writes 1 B (+1 B transposed)
            out.append((name, t.numel(), (6 if qT is not None else 5) * t.numel(), call))
        return out


def gemm_traffic(M_N_K_ok=True):
    digest = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]
    if not M_N_K_ok or GEMM_TRAFFIC is None or digest != GEMM_TRAFFIC["gemm_src_sha256_16"]:
        return None
    return 1024.0 * (GEMM_TRAFFIC["fetch_kib"] * GEMM_TRAFFIC["fetch_factor"] +
                     GEMM_TRAFFIC["write_kib"] * GEMM_TRAFFIC["write_factor"])


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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    F.lib()
    T = Timer(torch, stream)

    if args.hbm_only:
        hbm, hbm_kern = hbm_passes(np, torch, F, dev, T)
        print(json.dumps({"hbm_scale": hbm, "hbm_kernels_us": hbm_kern}), flush=True)
        return
    if args.square_only:
        print(json.dumps({"square_layer": square_layer(np, torch, F, dev, stream, T, args)}), flush=True)
        return

    mlp = MlpStep(np, torch, F, dev, layout=args.layout)
    log(f"timing {args.steps} steps of the MLP block")
    ms_per_step, wall, spread = timed_steps(torch, stream, mlp.step, args.steps, args.warmup)
    gemm_flops = sum(2.0 * L.M * L.N * L.K for L in mlp.lin.values()) * 3
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    log("per-kernel timings on the step's operands")
    gemm_us = {name: T.run(call, args.reps) for name, fl, call in mlp.gemms()}
    gemm_fl = {name: fl for name, fl, _ in mlp.gemms()}
    cast = {}
    for name, n, nbytes, call in mlp.casts():
        us = T.run(call, args.reps)
        cast[name] = {"elements": n, "bytes": nbytes, "transposed_copy": nbytes == 6 * n,
                      "amax_plus_cast_us": round(us, 2),
                      "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    torch.cuda.empty_cache()
    upd_us = T.run(lambda: F.amp_update_scale(mlp.scale, mlp.tracker, mlp.found, 2.0, 0.5, 2000),
                   args.reps)
    sum_gemm = sum(gemm_us.values())
    achieved = sum(gemm_fl.values()) / (sum_gemm * 1e-6) / 1e12
    cast_bytes = sum(c["bytes"] for c in cast.values())
    # x is cast once per step although gate and up both consume it
    sum_cast = sum(c["amax_plus_cast_us"] for c in cast.values())

    # ---- sampled check of the step's outputs against the oracle (after one
    # step from the initial loss scale, as timed)
    check = None
    if not args.no_check:
        log("sampled oracle check of the MLP step")
        mlp.scale.fill_(LOSS_SCALE)
        mlp.tracker.zero_()
        mlp.found.zero_()
        mlp.step()
        torch.cuda.synchronize()
        check = mlp_check(np, torch, F, mlp)

    side = {}
    if not args.no_side:
        side["square_layer"] = square_layer(np, torch, F, dev, stream, T, args)
        side["small_layer"] = small_layer(torch, F, dev, stream, T)
        log("MLP block through the PyTorch layer")
        side["mlp_block_autograd"] = mlp_autograd(torch, F, dev, stream)
    mlp_tr = sorted(mlp.tr)
    layout_used, inputs = mlp.layout, (mlp.host, mlp.dev)
    del mlp
    torch.cuda.empty_cache()
    if not args.no_side:
        side["mlp_copy_layouts"] = copy_layouts(np, torch, F, dev, stream, T, args, layout_used,
                                                inputs)
    del inputs
    torch.cuda.empty_cache()

    hbm, hbm_kern = ({}, {}) if args.no_hbm else hbm_passes(np, torch, F, dev, T)

    cpu = None
    if not args.no_cpu_baseline:
        log("oracle CPU baseline (a token slab of the MLP step)")
        cpu = cpu_baseline(np)

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
        "config": {"workload": "transformer MLP block T=8192 H=4096 F=14336 in FP8: gate, up, "
                               "down linears fwd+dgrad+wgrad (9 GEMMs), per-tensor dynamic "
                               "scaling of every operand, " + (
                                   "fused transposed copies of " + ", ".join(mlp_tr) +
                                   " read row-major by the weight-gradient GEMMs, every other "
                                   "backward operand read contraction-major, "
                                   if mlp_tr else
                                   "no transposed copies: dgrad/wgrad read the codes "
                                   "contraction-major, ") +
                               "GradScaler unscale/check fused into the dgrad/wgrad epilogues, "
                               "device-side scale update",
                   "tokens": 8192, "hidden": 4096, "ffn": 14336,
                   "x_h": "bf16 N(0,1)", "W": "bf16 N(0,0.02)",
                   "gy": "bf16 N(0,1e-4) x loss scale 65536", "y": "bf16", "grads": "fp16",
                   "formats": "e4m3fn x/h/W, e5m2 gy"},
        "step_pct_of_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "step_spread": spread,
        "step_breakdown_us": {"gemms": round(sum_gemm, 1), "casts_amax_quant": round(sum_cast, 1),
                              "update": round(upd_us, 2),
                              "sum": round(sum_gemm + sum_cast + upd_us, 1),
                              "step": round(1e3 * ms_per_step, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": gemm_traffic(),
                     "traffic_unit": "bytes per launch from L2 to the memory fabric (Infinity Cache "
                                     "or HBM), mean over the 9 GEMMs, counter-measured",
                     "kernel": "k_gemm_pingpong: the step's 9 GEMMs, 2*M*N*K flops each, "
                               "sum of flops / sum of mean launch times"},
        "gemms": {k: {"us": round(v, 2), "TFLOPs": round(gemm_fl[k] / (v * 1e-6) / 1e12, 1),
                      "frac": round(gemm_fl[k] / (v * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4)}
                  for k, v in gemm_us.items()},
        "casts": cast,
        "casts_GBps": round(cast_bytes / (sum_cast * 1e-6) / 1e9, 1),
        "casts_hbm_frac": round(cast_bytes / (sum_cast * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "hbm_scale": {k: (round(v, 1) if isinstance(v, float) else v) for k, v in hbm.items()},
        "hbm_frac": {k[:-5]: round(v / PEAK_HBM_GBPS, 4) for k, v in hbm.items()
                     if k.endswith("_GBps")},
        "hbm_kernels_us": {k: round(v, 2) for k, v in hbm_kern.items()},
        "wall_s_timed_region": round(wall, 4),
        "check": check,
        "cpu_baseline": cpu,
    }
    out.update(side)
    print(json.dumps(out), flush=True)


def mlp_check(np, torch, F, mlp, n_pts=256):
    """Recompute every cast with the oracle from the same host inputs and
    compare codes, transposed codes and records bit for bit; check sampled
    outputs of all nine GEMMs (forward bf16, unscaled fp16 gradients)."""
    import oracle as O
    from tests.parity import assert_codes_equal, check_gemm_values, check_unscaled_values
    H = mlp.host
    q = {"x": O.to_fp8(H["x"], O.E4M3FN), "h": O.to_fp8(H["h"], O.E4M3FN)}
    for n in mlp.NAMES:
        q["w_" + n] = O.to_fp8(H["w_" + n], O.E4M3FN)
        q["gy_" + n] = O.to_fp8(H["gy_" + n], O.E5M2)
    sv, ws = mlp.saved, mlp.ws
    pairs = [(sv["gate"].x_q, sv["gate"].x_qT, sv["gate"].x_sc, "x", O.E4M3FN),
             (sv["down"].x_q, sv["down"].x_qT, sv["down"].x_sc, "h", O.E4M3FN)]
    for n in mlp.NAMES:
        pairs.append((sv[n].w_q, sv[n].w_qT, sv[n].w_sc, "w_" + n, O.E4M3FN))
        pairs.append((ws[n].gy_q, ws[n].gy_qT, ws[n].gy_sc, "gy_" + n, O.E5M2))
    for dq, dqT, rec, key, fmt in pairs:
        assert_codes_equal(fmt, dq.cpu().numpy(), q[key].q, key)
        if dqT is not None:
            assert_codes_equal(fmt, dqT.cpu().numpy(), q[key].qT, key + " T")
        r = rec.read()
        assert r["amax_bits"] == q[key].sc.amax_bits and r["inv"] == q[key].sc.inv, key
    assert int(mlp.found.item()) == 0
    rng = np.random.default_rng(0)
    nw_max = 0.0
    u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    for n in mlp.NAMES:
        xk = "h" if n == "down" else "x"
        xq, wq, gq = q[xk], q["w_" + n], q["gy_" + n]
        for what, A, fa, B, ia, ib, got, fmt in (
                ("fwd", xq.q, O.E4M3FN, wq.q, xq.sc.inv, wq.sc.inv, mlp.y[n], O.BF16),
                ("dgrad", gq.q, O.E5M2, wq.qT, gq.sc.inv, wq.sc.inv, mlp.gx[n], O.F16),
                ("wgrad", gq.qT, O.E5M2, xq.qT, gq.sc.inv, xq.sc.inv, mlp.gw[n], O.F16)):
            M, Nn = A.shape[0], B.shape[0]
            ii, jj = rng.integers(0, M, n_pts), rng.integers(0, Nn, n_pts)
            c_ref = O.gemm_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
            ad = O.gemm_absdot_at(A, fa, B, O.E4M3FN, ia, ib, ii, jj)
            g = O.decode(fmt, u16(got)[ii, jj])
            if fmt == O.F16:
                nw = check_unscaled_values(u16(got)[ii, jj], c_ref, ad, A.shape[1], LOSS_SCALE,
                                           f"{n} {what}")
            else:
                nw = check_gemm_values(g, c_ref, ad, A.shape[1], fmt, f"{n} {what}")
            nw_max = max(nw_max, nw)
    return {"codes_and_records": "bit-exact (8 casts; transposed copies of " + (
                ", ".join(sorted(mlp.tr)) or "none") + ")",
            "found_inf": 0, "gemm_samples_per_gemm": n_pts, "gemms": 9, "ok": True,
            "max_abs_err_over_max_abs": float(nw_max)}


def square_layer(np, torch, F, dev, stream, T, args):
    """The square 4096^3 layer: fwd + bwd with fused unscale + update, and its
    three GEMMs' rate; also the same step with delayed and row-wise scaling."""
    import workloads as W
    from workloads.configs import SQUARE as S
    M, N, K = S.M, S.N, S.K
    log("square layer")
    x = bf16_dev(torch, np, S.x(), dev)
    w = bf16_dev(torch, np, S.w(), dev)
    gy = bf16_dev(torch, np, loss_scaled(np, S.gy()), dev)
    # the transposed copies fp8_linear_copies picks (gy's alone at this size)
    xt, wt, gt = F.fp8_linear_copies(M, N, K)
    saved = F.LinearSaved(M, N, K, device=dev, x_transposed=xt, w_transposed=wt)
    ws = F.LinearBwdWs(M, N, device=dev, transposed=gt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gx = torch.empty((M, K), dtype=torch.float16, device=dev)
    gw = torch.empty((N, K), dtype=torch.float16, device=dev)
    scale = torch.tensor([LOSS_SCALE], dtype=torch.float32, device=dev)
    tracker = torch.zeros(1, dtype=torch.int32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    steps = max(args.steps, 20)
    ms, _, _ = timed_steps(torch, stream, step, steps, args.warmup)
    fl = 2.0 * M * N * K
    # the three GEMMs as the backward runs them: a missing copy's operand read
    # contraction-major
    wk, gk, xk = not wt, not gt, not xt
    g = [T.run(lambda: F.fp8_gemm(saved.x_q, F.E4M3FN, saved.w_q, F.E4M3FN, saved.x_sc.inv_ptr(),
                                  saved.w_sc.inv_ptr(), y, F.OUT_BF16), args.reps),
         T.run(lambda: F.fp8_gemm_kmajor_unscale(
             ws.gy_q, F.E5M2, 0, saved.w_q if wk else saved.w_qT, F.E4M3FN, wk,
             ws.gy_sc.inv_ptr(), saved.w_sc.inv_ptr(), scale, found, gx), args.reps),
         T.run(lambda: F.fp8_gemm_kmajor_unscale(
             ws.gy_q if gk else ws.gy_qT, F.E5M2, gk, saved.x_q if xk else saved.x_qT, F.E4M3FN, xk,
             ws.gy_sc.inv_ptr(), saved.x_sc.inv_ptr(), scale, found, gw), args.reps)]
    rec = F.ScaleRec(device=dev)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    qT = torch.empty((K, M), dtype=torch.uint8, device=dev) if xt else None
    c_us = T.run(lambda: (F.fp8_amax(x, rec), F.fp8_quantize(x, F.E4M3FN, rec, q, qT)), args.reps)
    gavg = sum(g) / 3
    out = {"workload": "square linear 4096^3 (x with 0.1% outliers x50), fwd + bwd with fused "
                       "unscale + update",
           "transposed_copies": [k for k, v in (("x", xt), ("w", wt), ("gy", gt)) if v],
           "ms_per_step": round(ms, 4), "TFLOPs": round(3 * fl / (ms * 1e-3) / 1e12, 1),
           "gemm_us": [round(v, 2) for v in g],
           "gemm_frac": round(fl / (gavg * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
           "cast_x_amax_quant_us": round(c_us, 2)}
    # the same step with every transposed copy
    saved_a, ws_a = F.LinearSaved(M, N, K, device=dev), F.LinearBwdWs(M, N, device=dev)

    def step_all_copies():
        F.fp8_scaled_linear_fwd(x, w, saved_a, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_unscale(gy, saved_a, ws_a, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    ms_a, _, _ = timed_steps(torch, stream, step_all_copies, steps, args.warmup)
    out["all_copies_ms_per_step"] = round(ms_a, 4)
    del saved_a, ws_a
    # the same step with delayed scaling of x, W and gy (history of 16)
    hx, hw, hg = (torch.ones(16, dtype=torch.float32, device=dev) for _ in range(3))

    def step_delayed():
        F.fp8_scaled_linear_fwd_delayed(x, w, saved, hx, hw, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_delayed_unscale(gy, saved, ws, hg, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    ms_d, _, _ = timed_steps(torch, stream, step_delayed, steps, args.warmup)
    out["delayed_scaling_ms_per_step"] = round(ms_d, 4)
    saved_rw, ws_rw = F.LinearSavedRW(M, N, K, device=dev), F.LinearBwdWsRW(M, N, device=dev)

    def step_rowwise():
        F.fp8_scaled_linear_fwd_rowwise(x, w, saved_rw, y, F.OUT_BF16)
        F.fp8_scaled_linear_bwd_rowwise_unscale(gy, saved_rw, ws_rw, scale, found, gx, gw)
        F.amp_update_scale(scale, tracker, found, 2.0, 0.5, 2000)

    ms_r, _, _ = timed_steps(torch, stream, step_rowwise, steps, args.warmup)
    out["rowwise_scaling_ms_per_step"] = round(ms_r, 4)
    return out


def hbm_passes(np, torch, F, dev, T):
    """Memory-bound kernels at HBM scale (working sets far above the 256 MB
    Infinity Cache), logical bytes: the quantize workload (2^28 bf16 elements,
    e4m3 with magnitudes 10^U(-6,3) and e5m2 with 10^U(-8,-2)), the same tensor
    as a 16384 x 16384 matrix cast with its transposed copy (per-tensor and
    row-wise), and the GradScaler workload's unscale pass over 200 fp16
    tensors."""
    from workloads import configs as C
    hbm, kern = {}, {}
    log("HBM-scale quantize passes")
    big = torch.from_numpy(C.quant_act().view(np.int16)).view(torch.bfloat16).to(dev)
    nb = big.numel()
    bq = torch.empty(big.shape, dtype=torch.uint8, device=dev)
    brec = F.ScaleRec(device=dev)
    kern["amax_2p28"] = T.run(lambda: F.fp8_amax(big, brec), 10)
    kern["quantize_2p28"] = T.run(lambda: F.fp8_quantize(big, F.E4M3FN, brec, bq), 10)
    hbm["amax_GBps"] = 2.0 * nb / (kern["amax_2p28"] * 1e-6) / 1e9
    hbm["quantize_GBps"] = 3.0 * nb / (kern["quantize_2p28"] * 1e-6) / 1e9
    hbm["amax_plus_quantize_GBps"] = 5.0 * nb / ((kern["amax_2p28"] + kern["quantize_2p28"]) * 1e-6) / 1e9
    amax_big = float(np.array([brec.read()["amax_bits"]], np.uint32).view(np.float32)[0])
    bh = torch.full((16,), amax_big, dtype=torch.float32, device=dev)
    kern["quantize_delayed_2p28"] = T.run(lambda: F.fp8_quantize_delayed(big, F.E4M3FN, brec, bh, bq), 10)
    hbm["quantize_delayed_GBps"] = 3.0 * nb / (kern["quantize_delayed_2p28"] * 1e-6) / 1e9
    # the same elements as a 16384 x 16384 matrix with its transposed copy:
    # amax (2 B/el) + cast (2 B read, 1 + 1 B written)
    side = 1 << 14
    big2 = big.view(side, side)
    bqT = torch.empty((side, side), dtype=torch.uint8, device=dev)
    bq2 = bq.view(side, side)
    kern["quantize_transpose_16384sq"] = T.run(lambda: F.fp8_quantize(big2, F.E4M3FN, brec, bq2, bqT), 10)
    hbm["quantize_transpose_GBps"] = 4.0 * nb / (kern["quantize_transpose_16384sq"] * 1e-6) / 1e9
    hbm["amax_plus_quantize_transpose_GBps"] = 6.0 * nb / (
        (kern["amax_2p28"] + kern["quantize_transpose_16384sq"]) * 1e-6) / 1e9
    brs, bcs = F.RowScalesDev(side, device=dev), F.RowScalesDev(side, device=dev)
    kern["quantize_rowwise_transpose_16384sq"] = T.run(
        lambda: F.fp8_quantize_rowwise(big2, F.E4M3FN, brs, bq2, bcs, bqT), 10)
    hbm["quantize_rowwise_transpose_GBps"] = 6.0 * nb / (kern["quantize_rowwise_transpose_16384sq"] * 1e-6) / 1e9
    del big, bq, bh, big2, bqT, bq2
    gbig = torch.from_numpy(C.quant_grad().view(np.int16)).view(torch.bfloat16).to(dev)
    gq = torch.empty(gbig.shape, dtype=torch.uint8, device=dev)
    grec = F.ScaleRec(device=dev)
    kern["amax_2p28_grad"] = T.run(lambda: F.fp8_amax(gbig, grec), 10)
    kern["quantize_e5m2_2p28"] = T.run(lambda: F.fp8_quantize(gbig, F.E5M2, grec, gq), 10)
    hbm["amax_plus_quantize_e5m2_GBps"] = 5.0 * nb / (
        (kern["amax_2p28_grad"] + kern["quantize_e5m2_2p28"]) * 1e-6) / 1e9
    del gbig, gq
    log("HBM-scale unscale pass")
    sizes = C.scaler_sizes()
    grads = [(torch.randn(int(n), device=dev) * 0.5).half() for n in sizes]
    one = torch.ones(1, dtype=torch.float32, device=dev)
    fz = torch.zeros(1, dtype=torch.int32, device=dev)
    kern["unscale_check_200_tensors"] = T.run(lambda: F.amp_unscale_check(grads, one, fz), 10)
    ng = int(sizes.sum())
    hbm["unscale_GBps"] = 4.0 * ng / (kern["unscale_check_200_tensors"] * 1e-6) / 1e9
    hbm["unscale_elements"] = ng
    nws = torch.empty(F.amp_norm_workspace_len([g.numel() for g in grads]), dtype=torch.float32,
                      device=dev)
    nout = torch.empty(2, dtype=torch.float32, device=dev)
    kern["unscale_check_norm_200_tensors"] = T.run(
        lambda: F.amp_unscale_check_norm(grads, one, fz, nws, nout), 10)
    hbm["unscale_norm_GBps"] = 4.0 * ng / (kern["unscale_check_norm_200_tensors"] * 1e-6) / 1e9
    del grads, nws
    torch.cuda.empty_cache()
    return hbm, kern


def small_layer(torch, F, dev, stream, T, reps=200):
    """The small layer (B=64, K=128, N=256): launch-latency bound, so its
    time per phase and its kernel launches are reported, eager and replayed
    from a HIP graph."""
    from workloads.configs import SMALL as S
    import numpy as np
    x, w, gy = (bf16_dev(torch, np, a, dev) for a in (S.x(), S.w(), S.gy()))
    # the copies fp8_linear_copies picks: none for a layer this small, so each
    # pass runs in one launch (casts fused into the GEMM blocks)
    xt, wt, gt = F.fp8_linear_copies(S.M, S.N, S.K)
    saved = F.LinearSaved(S.M, S.N, S.K, device=dev, x_transposed=xt, w_transposed=wt)
    ws = F.LinearBwdWs(S.M, S.N, device=dev, transposed=gt)
    one_launch = not (xt or wt or gt)
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
        return round(T.run(g.replay, reps), 2)

    out = {"workload": "small linear B=64 K=128 N=256 + GradScaler step (init 65536, "
                       "interval 2000)",
           "fwd_us": round(T.run(fwd, reps), 2),
           "bwd_us": round(T.run(bwd, reps), 2),
           "scaler_step_us": round(T.run(scaler, reps), 2),
           "step_us": round(T.run(step, reps), 2),
           "step_fused_unscale_us": round(T.run(step_fused, reps), 2),
           # without transposed copies each pass is one launch (every GEMM
           # block reduces and casts what it needs); with them, tensors of at
           # most 64 Ki elements are cast by one block each and the two
           # backward GEMMs share a launch
           "transposed_copies": [k for k, v in (("x", xt), ("w", wt), ("gy", gt)) if v],
           "launches": ({"fwd": 1, "bwd": 1, "scaler_step": 2, "step_fused_unscale": 3}
                        if one_launch else
                        {"fwd": 2, "bwd": 2, "scaler_step": 2, "step_fused_unscale": 5})}
    out["step_graph_replay_us"] = replay_us(step)
    out["step_fused_unscale_graph_replay_us"] = replay_us(step_fused)
    out["TFLOPs_eager"] = round(3 * 2.0 * S.M * S.N * S.K / (out["step_us"] * 1e-6) / 1e12, 4)
    return out


def copy_layouts(np, torch, F, dev, stream, T, args, used, inputs):
    """The MLP step with the other transposed-copy layouts, on the same inputs,
    for comparison with the headline's: step time and the nine GEMMs' fraction
    of FP8 peak."""
    out = {"headline_layout": used}
    for layout in ("auto", "none", "all"):
        if layout == used:
            continue
        log(f"MLP step with the '{layout}' copy layout")
        m = MlpStep(np, torch, F, dev, layout=layout, inputs=inputs)
        ms, _, _ = timed_steps(torch, stream, m.step, args.steps, args.warmup)
        g = [(fl, T.run(call, args.reps)) for _, fl, call in m.gemms()]
        frac = sum(fl for fl, _ in g) / (sum(us for _, us in g) * 1e-6) / 1e12 / PEAK_FP8_TFLOPS
        out[layout] = {"copies": sorted(m.tr), "ms_per_step": round(ms, 4), "gemm_frac": round(frac, 4)}
        del m
        torch.cuda.empty_cache()
    return out


def mlp_autograd(torch, F, dev, stream, steps=10, warmup=3):
    """The MLP block's three linears trained through Float8Linear and autograd
    (each module casts its own input), device data at the block's shapes."""
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

    for _ in range(warmup):
        autograd_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        autograd_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 9 * 2.0 * T * Fd * H
    return {"workload": "MLP block T=8192 H=4096 F=14336 through Float8Linear + autograd "
                        "(bf16 grads, x cast by each of gate and up)",
            "ms_per_step": round(ms, 4), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1)}


def cpu_baseline(np, tokens=512):
    """The oracle (plain C, OpenMP) on the host cores, running the MLP step on
    a slab of `tokens` of the 8192 tokens (full weights): the eight casts with
    transposed copies, the nine GEMMs (fp32 sequential accumulation), the
    unscale/check of the six fp16 gradients and the update.  Throughput in the
    metric's unit: the slab's GEMM flops over the slab step's wall time."""
    import oracle as O
    import workloads as W
    from workloads.configs import mlp_linear
    lin = {n: mlp_linear(n) for n in ("gate", "up", "down")}
    # the slab: the first `tokens` rows of x, h and the gradients (the generator
    # is keyed by element index, so these are the full tensors' first rows)
    rows = lambda L, stream, cols, sigma: W.normal_bf16(L.seed, L.streams[stream], (tokens, cols), sigma)
    x = rows(lin["gate"], 0, lin["gate"].K, lin["gate"].x_sigma)
    h = rows(lin["down"], 0, lin["down"].K, lin["down"].x_sigma)
    w = {n: lin[n].w() for n in lin}
    gy = {n: loss_scaled(np, rows(lin[n], 2, lin[n].N, lin[n].gy_sigma)) for n in lin}
    t0 = time.perf_counter()
    xq, hq = O.to_fp8(x, O.E4M3FN), O.to_fp8(h, O.E4M3FN)
    flops = 0.0
    grads = []
    for n in lin:
        iq = hq if n == "down" else xq
        wq = O.to_fp8(w[n], O.E4M3FN)
        gq = O.to_fp8(gy[n], O.E5M2)
        O.round_out(O.gemm(iq.q, O.E4M3FN, wq.q, O.E4M3FN, iq.sc.inv, wq.sc.inv), O.BF16)
        grads.append(O.round_out(O.gemm(gq.q, O.E5M2, wq.qT, O.E4M3FN, gq.sc.inv, wq.sc.inv), O.F16))
        grads.append(O.round_out(O.gemm(gq.qT, O.E5M2, iq.qT, O.E4M3FN, gq.sc.inv, iq.sc.inv), O.F16))
        L = lin[n]
        flops += 3 * 2.0 * tokens * L.N * L.K
    found = O.unscale_check(grads, LOSS_SCALE, 0)
    O.update_scale(O.ScalerState(np.float32(LOSS_SCALE), 0), found, 2.0, 0.5, 2000)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"the MLP step on {tokens} of 8192 tokens (full weights): 8 casts with "
                      f"transposed copies, 9 GEMMs ({flops / 1e9:.0f} GFLOP, fp32 sequential "
                      f"accumulation), unscale/check of 6 fp16 gradients, update; {dt:.2f} s wall"}


if __name__ == "__main__":
    main()
