"""amp_unscale_check_norm_noalloc (the no-allocation variant of
amp_unscale_check_norm, for callers that cannot allocate device memory)
against amp_unscale_check_norm with a caller workspace: the same unscaled
gradients, flag and (sum of squares, norm), bit for bit, on two calls in a
row, the second smaller than the first (the scratch keeps the first call's
contents, none of which may leak into the second)."""
import ctypes

import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def f16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.float16).to(DEV)


def both(grads_bits, scale_val):
    """The same list through the workspace entry point and the no-allocation
    one, each on its own copy of the gradients."""
    a = [f16_dev(g) for g in grads_bits]
    b = [f16_dev(g) for g in grads_bits]
    scale = torch.tensor([scale_val], dtype=torch.float32, device=DEV)
    fa = torch.zeros(1, dtype=torch.int32, device=DEV)
    fb = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(F.amp_norm_workspace_len([g.numel() for g in a]), dtype=torch.float32,
                     device=DEV)
    na = torch.empty(2, dtype=torch.float32, device=DEV)
    nb = torch.full((2,), -1.0, dtype=torch.float32, device=DEV)
    F.amp_unscale_check_norm(a, scale, fa, ws, na)
    F.amp_unscale_check_norm_noalloc(b, scale, fb, nb)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert int(fa.item()) == int(fb.item())
    assert torch.equal(na.view(torch.int32), nb.view(torch.int32)), (na, nb)
    return int(fb.item()), nb.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    rng = np.random.default_rng(71)
    sizes = [int(n) for n in rng.integers(1, 3_000_000, 40)] + [8192 * 300 + 5, 7, 0]
    big = [W.normal_f16(71, i, (n,), 1e-5 * 65536.0) for i, n in enumerate(sizes)]
    f1, n1 = both(big, 65536.0)
    assert f1 == 0 and n1[0] > 0
    # second call: fewer, smaller tensors and a non-finite value; the scratch
    # still holds the first call's partial sums, which must not count
    small = [W.normal_f16(72, i, (n,), 3.0) for i, n in enumerate([5000, 77, 123_457])]
    f2, n2 = both(small, 8.0)
    assert f2 == 0 and n2[0] > 0
    small[1][10] = 0x7C00
    f3, n3 = both(small, 8.0)
    assert f3 == 1 and np.isinf(n3[0])


def test_noalloc_rejects_oversize_list_before_any_launch():
    L = F.lib()
    # 1.1e10 elements need more slots than the scratch holds: FP8SG_ERR_SHAPE (2),
    # returned before any pointer is used
    n = 11 * 10 ** 9 // 8
    ptrs = (ctypes.c_void_p * 8)(*([0x10000] * 8))
    numel = (ctypes.c_int64 * 8)(*([n] * 8))
    scale = torch.ones(1, dtype=torch.float32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.zeros(2, dtype=torch.float32, device=DEV)
    st = L.amp_unscale_check_norm_noalloc(ptrs, numel, 8, ctypes.c_void_p(scale.data_ptr()),
                                          ctypes.c_void_p(found.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr()), None)
    assert st == 2
    assert F.amp_norm_workspace_len([n] * 8) > F.NOALLOC_NORM_SLOTS
