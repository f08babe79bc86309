"""The whole training-step path (forward, backward, unscale + non-finite check,
scale update) enqueues only kernels on the caller's stream: no host
synchronisation, no allocation and no memset.  So it can be captured in a HIP
graph.  Each replay must reproduce the eager results bit for bit, including
after eager work on the same buffers between replays."""
import numpy as np
import pytest
import torch

import fp8_scaled_gemm_amd as F
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.contiguous().view(torch.uint8) if t.dtype != torch.uint8 else t


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("shape,copies", [((512, 768, 384), True), ((512, 768, 384), False),
                                          ((64, 256, 128), False)])
def test_step_graph_replay_matches_eager(fused, shape, copies):
    """With transposed copies; without them (the backward GEMMs read the codes
    contraction-major); and the small layer's one-launch passes."""
    M, N, K = shape
    x = torch.from_numpy(W.normal_bf16(41, 0, (M, K), 1.0).view(np.int16)).view(
        torch.bfloat16).to(DEV)
    w = torch.from_numpy(W.normal_bf16(41, 1, (N, K), 0.02).view(np.int16)).view(
        torch.bfloat16).to(DEV)
    gy = torch.from_numpy(W.normal_bf16(41, 2, (M, N), 1e-4 * 65536.0).view(
        np.int16)).view(torch.bfloat16).to(DEV)
    saved = F.LinearSaved(M, N, K, device=DEV, transposed=copies)
    ws = F.LinearBwdWs(M, N, device=DEV, transposed=copies)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gx = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gw = torch.empty((N, K), dtype=torch.float16, device=DEV)
    scale = torch.tensor([65536.0], device=DEV)
    tracker = torch.zeros(1, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step():
        F.fp8_scaled_linear_fwd(x, w, saved, y, F.OUT_BF16)
        if fused:  # unscale + check in the backward GEMMs' epilogues
            F.fp8_scaled_linear_bwd_unscale(gy, saved, ws, scale, found, gx, gw)
        else:
            F.fp8_scaled_linear_bwd(gy, saved, ws, gx, gw, F.OUT_F16)
            F.amp_unscale_check([gx, gw], scale, found)
        # growth factor 1: the tracker counts and resets, the scale (and so every
        # output) stays that of the eager reference step
        F.amp_update_scale(scale, tracker, found, 1.0, 0.5, 3)

    outs = [t for t in (y, gx, gw, saved.x_q, saved.x_qT, saved.w_q, saved.w_qT, saved.recs, ws.gy_q,
                        ws.gy_qT, ws.gy_sc.buf) if t is not None]
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    # one eager step has run (tracker 1); the interval is 3
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # tracker 2
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()  # captured, not run
    expect_scale, expect_tracker = 65536.0, 2
    for r in range(4):
        for t in (y, gx, gw, saved.x_q, ws.gy_q):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(e)), f"replay {r}"
        expect_tracker += 1
        if expect_tracker >= 3:
            expect_tracker = 0
        assert scale.item() == expect_scale and tracker.item() == expect_tracker, f"replay {r}"
        assert found.item() == 0
