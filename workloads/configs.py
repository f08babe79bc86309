"""The five synthetic workloads, with their seeds and tensor streams.

Shapes and distributions follow the workload list of this project: a small
FP8 linear layer with one GradScaler step, a square 4096^3 layer, a
transformer MLP block, a memory-bound quantize pass and a multi-tensor
GradScaler run.  "N(0, s)" means standard deviation s.  Each tensor has a
fixed (seed, stream) pair, so any element can be regenerated on its own.
"""
from dataclasses import dataclass, field

import numpy as np

from . import logmag_bf16, normal_bf16, normal_f32, f32_to_f16_bits, uniform

# GradScaler defaults [PT-CH20 §20.5.33]
INIT_SCALE = 65536.0
GROWTH = 2.0
BACKOFF = 0.5
INTERVAL = 2000


@dataclass
class Linear:
    """One FP8 linear layer: x [M,K], W [N,K], gy [M,N] (bf16 bit patterns)."""
    name: str
    M: int
    N: int
    K: int
    seed: int
    x_sigma: float
    w_sigma: float
    gy_sigma: float
    x_outlier_p: float = 0.0
    x_outlier_mult: float = 1.0
    streams: tuple = (1, 2, 3)

    def x(self):
        return normal_bf16(self.seed, self.streams[0], (self.M, self.K), self.x_sigma,
                           self.x_outlier_p, self.x_outlier_mult)

    def w(self):
        return normal_bf16(self.seed, self.streams[1], (self.N, self.K), self.w_sigma)

    def gy(self):
        return normal_bf16(self.seed, self.streams[2], (self.M, self.N), self.gy_sigma)

    def flops(self):
        return 3 * 2 * self.M * self.N * self.K


# Config 1: B=64, K=128, N=256; x ~N(0,1), W ~N(0,0.02), gy ~N(0,1e-3); seed 1.
SMALL = Linear("small linear B=64 K=128 N=256", M=64, N=256, K=128, seed=1,
               x_sigma=1.0, w_sigma=0.02, gy_sigma=1e-3)

# Config 2: B=K=N=4096; x ~N(0,1) with 0.1% outliers x50, W ~N(0,0.02),
# gy ~N(0,1e-4); seed 2.
SQUARE = Linear("square linear 4096x4096x4096", M=4096, N=4096, K=4096, seed=2,
                x_sigma=1.0, w_sigma=0.02, gy_sigma=1e-4, x_outlier_p=1e-3,
                x_outlier_mult=50.0)

# Config 3: transformer MLP block, tokens 8192, hidden 4096, ffn 14336.  Three
# linears (gate, up: [14336,4096]; down: [4096,14336]); activations ~N(0,1),
# weights ~N(0,0.02), grads ~N(0,1e-4); seed 3.  x is shared by gate and up.
MLP_T, MLP_H, MLP_F = 8192, 4096, 14336
MLP_SEED = 3
MLP = {
    # name: (M, N, K, stream of input, stream of weight, stream of grad)
    "gate": (MLP_T, MLP_F, MLP_H, 1, 2, 5),
    "up": (MLP_T, MLP_F, MLP_H, 1, 3, 6),
    "down": (MLP_T, MLP_H, MLP_F, 4, 7, 8),
}


def mlp_linear(name: str) -> Linear:
    M, N, K, sx, sw, sg = MLP[name]
    return Linear(f"MLP {name} T={MLP_T} H={MLP_H} F={MLP_F}", M=M, N=N, K=K, seed=MLP_SEED,
                  x_sigma=1.0, w_sigma=0.02, gy_sigma=1e-4, streams=(sx, sw, sg))


# Config 4: memory-bound quantize pass: 2^28 bf16 elements with magnitudes
# 10^U(-6,3) and random sign (-> e4m3), plus an equal-size gradient tensor at
# 10^U(-8,-2) (-> e5m2); seed 4.
QUANT_N = 268_435_456
QUANT_SEED = 4


def quant_act(n=QUANT_N):
    return logmag_bf16(QUANT_SEED, 1, (n,), -6.0, 3.0)


def quant_grad(n=QUANT_N):
    return logmag_bf16(QUANT_SEED, 2, (n,), -8.0, -2.0)


# Config 5: GradScaler over 200 fp16 gradients, sizes log-uniform in
# [4096, 67108864], values N(0,1e-5) * scale, 1000 steps, an inf/NaN injected
# into one random tensor with probability 0.01 per step; growth interval 100,
# growth 2, backoff 0.5; seed 5.
SCALER_SEED = 5
SCALER_NT = 200
SCALER_STEPS = 1000
SCALER_P_INJECT = 0.01
SCALER_INTERVAL = 100
SCALER_SIGMA = 1e-5
INJECT_BITS = (0x7C00, 0xFC00, 0x7E00)  # fp16 +inf, -inf, NaN


def scaler_sizes(nt=SCALER_NT, lo=4096, hi=67108864, seed=SCALER_SEED):
    """floor(exp(U(ln lo, ln hi))) per tensor."""
    u = uniform(seed, 100, nt)
    return np.floor(np.exp(np.log(lo) + (np.log(hi) - np.log(lo)) * u)).astype(np.int64)


def scaler_grad(t: int, n: int, scale: float, seed=SCALER_SEED, step: int = 0):
    """fp16 bit patterns of fp16(N(0, 1e-5) * scale) for tensor t at a step."""
    v = normal_f32(seed, 1000 + t + 1_000_000 * step, n, SCALER_SIGMA * scale)
    return f32_to_f16_bits(v)


@dataclass
class Injection:
    step: int
    tensor: int
    index: int
    bits: int


def injection_schedule(sizes, steps=SCALER_STEPS, p=SCALER_P_INJECT, seed=SCALER_SEED):
    """Host-seeded schedule: at each step, with probability p, one of +inf,
    -inf, NaN at a uniform (tensor, index)."""
    nt = len(sizes)
    u = uniform(seed, 200, 4 * steps).reshape(steps, 4)
    out = []
    for s in range(steps):
        if u[s, 0] < p:
            t = int(u[s, 1] * nt)
            idx = int(u[s, 2] * int(sizes[t]))
            kind = int(u[s, 3] * 3)
            out.append(Injection(s, t, idx, INJECT_BITS[kind]))
    return out
