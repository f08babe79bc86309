"""fp8_quantize_from_amax: the cast with an amax the caller supplies
[FP8-TRAIN §2: scale = fp8_max / amax in fp64, then x * scale, clamp, cast].

The case it exists for is a tensor split across devices that must keep one
per-tensor scale: each shard reduces its own amax, the shards' amaxes are
combined by a MAX (an all-reduce across devices; on one GPU a device-side
maximum stands in for it), and every shard is cast with the combined amax.
The shards' codes and scale records must then equal the oracle's cast of the
whole tensor, bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
import workloads as W
from tests.parity import assert_codes_equal
from tests.test_gpu_kernels import dev_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def rec_amax(rec: F.ScaleRec) -> torch.Tensor:
    return rec.buf[:4].view(torch.float32)


def rec_fields_equal(rec: F.ScaleRec, ref: O.Scale, what=""):
    r = rec.read()
    assert r["amax_bits"] == ref.amax_bits, what
    if np.isnan(ref.scale):
        assert np.isnan(r["scale"]) and np.isnan(r["inv"]), what
        return
    got = np.array([r["scale"], r["inv"]], np.float64).view(np.uint64)
    want = np.array([ref.scale, ref.inv], np.float64).view(np.uint64)
    assert np.array_equal(got, want), (what, r, ref)
    assert r["scale32_bits"] == int(np.float32(ref.scale32).view(np.uint32)), what
    assert r["inv32_bits"] == int(np.float32(ref.inv32).view(np.uint32)), what


@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
@pytest.mark.parametrize("shape,split,with_t", [
    ((4096, 4096), (1536, 4096), True),    # tiled cast with transposed copy
    ((1024, 768), (96, 352, 1024), True),  # three shards
    ((1000, 777), (336, 1000), False),     # flat cast, ragged shard sizes
    ((1000, 777), (504, 1000), True),      # transposed copy of an odd shape (per-element path)
])
def test_row_shards_with_combined_amax_match_whole_tensor(fmt, shape, split, with_t):
    rows, cols = shape
    sigma = 1.0 if fmt == F.E4M3FN else 1e-4
    x = W.normal_bf16(61, fmt, shape, sigma, 1e-3, 50.0)
    ref = O.to_fp8(x, fmt, with_transpose=with_t)
    xd = dev_bf16(x).reshape(rows, cols)
    bounds = [0, *split]
    shards = [xd[a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    # each shard's own amax, then the MAX over shards on the device
    part = [F.ScaleRec() for _ in shards]
    for s, r in zip(shards, part):
        F.fp8_amax(s, r)
    amax = rec_amax(part[0]).clone()
    for r in part[1:]:
        amax = torch.maximum(amax, rec_amax(r))
    out = [F.ScaleRec() for _ in shards]
    qs = [torch.empty(s.shape, dtype=torch.uint8, device=DEV) for s in shards]
    qTs = [torch.empty((cols, s.shape[0]), dtype=torch.uint8, device=DEV) if with_t else None
           for s in shards]
    for s, r, q, qT in zip(shards, out, qs, qTs):
        F.fp8_quantize_from_amax(s, fmt, amax, r, q, qT)
    torch.cuda.synchronize()
    for k, r in enumerate(out):
        rec_fields_equal(r, ref.sc, f"shard {k}")
    assert_codes_equal(fmt, torch.cat(qs).cpu().numpy(), ref.q, "codes")
    if with_t:
        assert_codes_equal(fmt, torch.cat(qTs, dim=1).cpu().numpy(), ref.qT, "transposed codes")


@pytest.mark.parametrize("given", [2.5, 1e-30, 0.0, -3.0, float("inf"), float("nan"), 3.0e38])
@pytest.mark.parametrize("fmt", [F.E4M3FN, F.E5M2])
def test_given_amax_values(given, fmt):
    """The scale follows the given amax, whatever the record held before (here
    bytes of 0xAB): a negative amax counts as 0 and gives the EPS scale, NaN the
    NaN scale, +inf a zero scale (finite inputs cast to +-0)."""
    x = W.normal_bf16(62, 1, (64, 80), 1.0, 0.01, 100.0)
    xd = dev_bf16(x).reshape(64, 80)
    rec = F.ScaleRec(buf=torch.full((F.SCALE_REC_BYTES,), 0xAB, dtype=torch.uint8, device=DEV))
    amax = torch.tensor([given], dtype=torch.float32, device=DEV)
    q = torch.empty((64, 80), dtype=torch.uint8, device=DEV)
    qT = torch.empty((80, 64), dtype=torch.uint8, device=DEV)
    F.fp8_quantize_from_amax(xd, fmt, amax, rec, q, qT)
    torch.cuda.synchronize()
    bits = int(np.float32(given).view(np.uint32))
    if np.isnan(given):
        bits = 0x7FC00000
    elif given < 0:
        bits = 0
    sc = O.scale_from_amax(bits, fmt)
    rec_fields_equal(rec, sc, f"amax {given}")
    codes = O.quantize(x, fmt, sc.scale32)
    assert_codes_equal(fmt, q.cpu().numpy(), codes, f"amax {given}")
    assert_codes_equal(fmt, qT.cpu().numpy(), O.transpose(codes.reshape(64, 80)), f"amax {given} T")


def test_given_amax_equals_two_pass_cast():
    """With the tensor's own amax (read from fp8_amax's record) the codes and
    record equal fp8_amax + fp8_quantize's."""
    x = W.normal_bf16(63, 1, (512, 384), 1.0, 1e-3, 50.0)
    xd = dev_bf16(x).reshape(512, 384)
    r1, r2 = F.ScaleRec(), F.ScaleRec()
    q1, q2 = (torch.empty((512, 384), dtype=torch.uint8, device=DEV) for _ in range(2))
    t1, t2 = (torch.empty((384, 512), dtype=torch.uint8, device=DEV) for _ in range(2))
    F.fp8_amax(xd, r1)
    F.fp8_quantize(xd, F.E4M3FN, r1, q1, t1)
    F.fp8_quantize_from_amax(xd, F.E4M3FN, rec_amax(r1), r2, q2, t2)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(t1, t2)
    a, b = r1.read(), r2.read()
    for k in ("amax_bits", "scale32_bits", "inv32_bits", "scale", "inv"):
        assert a[k] == b[k], k
