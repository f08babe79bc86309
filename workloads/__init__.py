"""Seeded synthetic inputs shared by the oracle side and the HIP side.

Both sides read the very same host bits: the generator (``synth.c``) writes
fp32 values, which are rounded to bf16 with torch's CPU cast or to fp16 with
numpy's cast.  This module holds none of the FP8 method's arithmetic.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth.c")
LIB = os.path.join(HERE, "libsynth.so")

_lib = None


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-fvisibility=hidden", "-Wall", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        u64, i64, f64, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.syn_u64.argtypes = [u64, u64, i64, i64, P]
        L.syn_uniform_f64.argtypes = [u64, u64, i64, i64, P]
        L.syn_normal_f32.argtypes = [u64, u64, i64, i64, f64, f64, f64, P]
        L.syn_logmag_f32.argtypes = [u64, u64, i64, i64, f64, f64, P]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def u64(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().syn_u64(seed, stream, start, n, _p(out))
    return out


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().syn_uniform_f64(seed, stream, start, n, _p(out))
    return out


def normal_f32(seed, stream, n, sigma, outlier_p=0.0, outlier_mult=1.0, start=0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().syn_normal_f32(seed, stream, start, n, sigma, outlier_p, outlier_mult, _p(out))
    return out


def logmag_f32(seed, stream, n, lo10, hi10, start=0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().syn_logmag_f32(seed, stream, start, n, lo10, hi10, _p(out))
    return out


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with torch's CPU cast (round-to-nearest-even);
    returns the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 to fp16 with numpy's cast (round-to-nearest-even)."""
    return np.ascontiguousarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


_CHUNK = 1 << 25


def _chunked(gen, n, conv):
    out = np.empty(n, np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = conv(gen(s, m))
    return out


def normal_bf16(seed, stream, shape, sigma, outlier_p=0.0, outlier_mult=1.0) -> np.ndarray:
    """bf16 bit patterns of sigma * N(0,1) (sigma is the standard deviation),
    with an optional fraction outlier_p of elements multiplied by outlier_mult."""
    n = int(np.prod(shape))
    out = _chunked(lambda s, m: normal_f32(seed, stream, m, sigma, outlier_p, outlier_mult, s),
                   n, f32_to_bf16_bits)
    return out.reshape(shape)


def normal_f16(seed, stream, shape, sigma) -> np.ndarray:
    n = int(np.prod(shape))
    out = _chunked(lambda s, m: normal_f32(seed, stream, m, sigma, start=s), n, f32_to_f16_bits)
    return out.reshape(shape)


def logmag_bf16(seed, stream, shape, lo10, hi10) -> np.ndarray:
    """bf16 bit patterns of random-sign magnitudes 10^U(lo10, hi10)."""
    n = int(np.prod(shape))
    out = _chunked(lambda s, m: logmag_f32(seed, stream, m, lo10, hi10, s), n, f32_to_bf16_bits)
    return out.reshape(shape)
