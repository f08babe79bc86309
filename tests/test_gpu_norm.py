"""GPU parity for amp_unscale_check_norm: the unscaled gradients and the
non-finite flag bit-exact against the oracle's unscale, and the global
(sum of squares, 2-norm) against the oracle's exact sum.

Bound, from the kernel's arithmetic (u = 2^-24; every term is >= 0, so each
rounded addition adds at most u times the running total):
  - each square of a stored fp16 value is exact in fp32;
  - the <= 8 squares of one 16-byte load are added in order: <= 7 roundings;
  - a thread adds its 4 load sums in order: 3;
  - the wave's xor-shuffle tree: 6 roundings; the block adds 4 wave sums: 3;
  - the per-block fp32 sums are added in fp64 (error below 1e-11 relative
    here) and the total is rounded to fp32 once: 1.
So |sumsq - exact| <= 20 u * exact (to first order), and the square root,
taken in fp64 and rounded to fp32, is within 20/2 u + u of the exact norm."""
import math

import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import oracle as O
import workloads as W
from workloads import configs as C

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24
TOL_SUMSQ = 20 * U + 1e-11
TOL_NORM = 11 * U + 1e-11


def to_dev16(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(DEV)


def run_norm(dev_grads, scale):
    numels = [g.numel() for g in dev_grads]
    ws = torch.empty(max(F.amp_norm_workspace_len(numels), 1), dtype=torch.float32, device=DEV)
    out = torch.full((2,), -1.0, dtype=torch.float32, device=DEV)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.amp_unscale_check_norm(dev_grads, s, found, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), int(found.item())


def check_against_oracle(host_grads, scale, views_of=None):
    """host_grads: list of uint16 arrays; the device copies are views into one
    flat buffer at the given element offsets (or separate tensors)."""
    if views_of is None:
        dev = [to_dev16(g.copy()) for g in host_grads]
    else:
        flat = torch.zeros(views_of[-1] + 8, dtype=torch.float16, device=DEV)
        dev = []
        for g, off in zip(host_grads, views_of):
            v = flat[off:off + g.size]
            v.copy_(to_dev16(g.copy()))
            dev.append(v)
    got, found = run_norm(dev, scale)
    ref = [g.copy() for g in host_grads]
    ref_found = O.unscale_check(ref, np.float32(scale))
    for d, r in zip(dev, ref):
        assert np.array_equal(d.cpu().view(torch.int16).numpy().view(np.uint16), r)
    assert found == ref_found
    s_ref, n_ref = O.grad_norm(ref)
    if math.isnan(s_ref):
        assert math.isnan(got[0]) and math.isnan(got[1])
    elif math.isinf(s_ref):
        assert got[0] == math.inf and got[1] == math.inf
    else:
        assert abs(got[0] - s_ref) <= TOL_SUMSQ * s_ref, (got[0], s_ref)
        assert abs(got[1] - n_ref) <= TOL_NORM * n_ref, (got[1], n_ref)
    return got


def grads_for(sizes, seed, sigma=1e-5, scale=65536.0):
    return [W.normal_f16(seed, 100 + i, (n,), sigma * scale) for i, n in enumerate(sizes)]


@pytest.mark.parametrize("sizes", [[1], [8], [8192], [8193, 5, 100_000], [3, 0, 16_384 * 3 + 1],
                                   [70_000] * 70])
def test_norm_matches_oracle(sizes):
    check_against_oracle(grads_for(sizes, 5), 65536.0)


def test_norm_on_unaligned_views_of_one_buffer():
    sizes = [7, 8192, 13, 50_001, 1]
    offs, o = [], 1  # odd element offsets: 2-byte but not 16-byte aligned views
    for n in sizes:
        offs.append(o)
        o += n + 3
    offs.append(o)
    check_against_oracle(grads_for(sizes, 6), 1024.0, views_of=offs)


def test_norm_of_no_elements_is_zero():
    got, found = run_norm([torch.empty(0, dtype=torch.float16, device=DEV)], 2.0)
    assert got.tolist() == [0.0, 0.0] and found == 0
    got, found = run_norm([], 2.0)
    assert got.tolist() == [0.0, 0.0] and found == 0


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00])
def test_norm_with_a_nonfinite_gradient(bad):
    g = grads_for([5000, 300], 7)
    g[1][123] = bad
    check_against_oracle(g, 65536.0)


def test_norm_is_deterministic():
    host = grads_for([1_000_003, 77_777, 4096], 8)
    outs = []
    for _ in range(3):
        dev = [to_dev16(h.copy()) for h in host]
        outs.append(run_norm(dev, 65536.0)[0])
    assert all(np.array_equal(o.view(np.uint64), outs[0].view(np.uint64)) for o in outs)


def test_norm_at_the_gradscaler_workload_size():
    """One step of the 200-tensor GradScaler workload (about 1.7e9 elements)."""
    sizes = C.scaler_sizes()
    host = [C.scaler_grad(t, int(n), C.INIT_SCALE) for t, n in enumerate(sizes)]
    check_against_oracle(host, C.INIT_SCALE)
