"""Pins for the oracle's row-wise scaling ["FP8训练：量化、自动微分、Torchao", §1:
each row has its own scale factor, carried through the accumulation].  The
pins reduce it to the already pinned per-tensor path (a row alone, or rows of
equal magnitude), check the power-of-two closed forms of the vector-scaled
GEMM, and check the point of the method: rows of very different magnitudes
keep their precision, which a wrong axis or a shared scale would not."""
import numpy as np
import pytest

import oracle as O
import workloads as W


def f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(f):
    return W.f32_to_bf16_bits(np.asarray(f, np.float32)).reshape(np.shape(f))


def row_mags(seed, rows, cols, lo, hi):
    """rows with magnitudes 10^lo .. 10^hi (one decade step per row group)."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((rows, cols)) * (10.0 ** np.linspace(lo, hi, rows))[:, None]
    return to_bf16(f)


@pytest.mark.parametrize("fmt", [O.E4M3FN, O.E5M2])
def test_each_row_is_the_per_tensor_cast_of_that_row(fmt):
    x = row_mags(1, 12, 48, -4, 3)
    r = O.to_fp8_rowwise(x, fmt)
    for i in range(x.shape[0]):
        one = O.to_fp8(x[i:i + 1], fmt, with_transpose=False)
        assert np.array_equal(r.q[i], one.q[0])
        assert r.rows.amax_bits[i] == one.sc.amax_bits
        assert r.rows.scale[i] == one.sc.scale and r.rows.inv[i] == one.sc.inv
        assert r.rows.scale32[i] == one.sc.scale32
    # the transposed copy is the row-wise cast of the transposed tensor
    xT = np.ascontiguousarray(x.T)
    rt = O.to_fp8_rowwise(xT, fmt, with_transpose=False)
    assert np.array_equal(r.qT, rt.q) and np.array_equal(r.cols.inv, rt.rows.inv)


def test_equal_rows_reduce_to_per_tensor():
    base = W.normal_bf16(2, 0, (1, 64), 1.0)
    x = np.repeat(base, 16, axis=0)  # every row identical: same amax, same scale
    r = O.to_fp8_rowwise(x, O.E4M3FN)
    t = O.to_fp8(x, O.E4M3FN)
    assert np.array_equal(r.q, t.q)
    assert np.all(r.rows.inv == t.sc.inv)
    # the columns differ, so qT has per-column scales; each column's amax is its |value|
    assert np.array_equal(r.cols.amax_bits, O.amax_rows(np.ascontiguousarray(base.T)))


def test_power_of_two_row_changes_only_that_row():
    x = row_mags(3, 8, 32, -1, 1)
    y = x.copy()
    y[5] = to_bf16(f32(x[5]) * 2.0 ** 7)
    a, b = O.to_fp8_rowwise(x, O.E4M3FN), O.to_fp8_rowwise(y, O.E4M3FN)
    assert np.array_equal(a.q, b.q)  # codes unchanged, row 5 included
    assert np.array_equal(np.delete(a.rows.inv, 5), np.delete(b.rows.inv, 5))
    assert b.rows.inv[5] == a.rows.inv[5] * 2.0 ** 7 and b.rows.scale[5] == a.rows.scale[5] / 2 ** 7


def test_vector_gemm_closed_forms():
    rng = np.random.default_rng(4)
    A = rng.integers(0, 0x60, (24, 96)).astype(np.uint8)
    B = rng.integers(0, 0x60, (40, 96)).astype(np.uint8)
    base = O.gemm(A, O.E4M3FN, B, O.E4M3FN, 1.0, 1.0)
    # constant vectors are the per-tensor GEMM
    assert np.array_equal(O.gemm_vec(A, O.E4M3FN, B, O.E4M3FN, np.full(24, 0.375), np.full(40, 3.0)),
                          O.gemm(A, O.E4M3FN, B, O.E4M3FN, 0.375, 3.0))
    # powers of two scale each output exactly by inv_a[i] * inv_b[j]
    ia = 2.0 ** rng.integers(-6, 6, 24)
    ib = 2.0 ** rng.integers(-6, 6, 40)
    got = O.gemm_vec(A, O.E4M3FN, B, O.E4M3FN, ia, ib)
    assert np.array_equal(got, (base.astype(np.float64) * ia[:, None] * ib[None, :]).astype(np.float32))
    ii, jj = rng.integers(0, 24, 50), rng.integers(0, 40, 50)
    assert np.array_equal(O.gemm_vec_at(A, O.E4M3FN, B, O.E4M3FN, ia, ib, ii, jj), got[ii, jj])


def test_rowwise_keeps_every_rows_precision():
    """Rows spanning 10^-4 .. 10^2: with one scale per row every row of
    y = x W^T stays within FP8 precision of the exact product; one shared
    scale loses the small rows to the subnormal range."""
    x = row_mags(5, 32, 128, -4, 2)
    w = W.normal_bf16(5, 1, (64, 128), 0.05)
    exact = f32(x) @ f32(w).T
    rw = O.linear_fwd_rowwise(x, w).c.astype(np.float64)
    pt = O.linear_fwd(x, w).c.astype(np.float64)
    rel = lambda c: np.linalg.norm(c - exact, axis=1) / np.linalg.norm(exact, axis=1)
    assert np.all(rel(rw) < 0.1)
    assert rel(pt)[0] > 0.5  # the smallest row, cast with the largest row's scale


def test_rowwise_backward_uses_the_non_contraction_axes():
    x = row_mags(6, 48, 32, -2, 1)
    w = W.normal_bf16(6, 1, (16, 32), 0.1)
    gy = row_mags(7, 48, 16, -3, 0)
    fw = O.linear_fwd_rowwise(x, w)
    bw = O.linear_bwd_rowwise(gy, fw)
    ex_gx = f32(gy) @ f32(w)
    ex_gw = f32(gy).T @ f32(x)
    assert np.linalg.norm(bw.c_gx - ex_gx) / np.linalg.norm(ex_gx) < 0.15
    assert np.linalg.norm(bw.c_gw - ex_gw) / np.linalg.norm(ex_gw) < 0.15
    assert bw.gy.rows.inv.size == 48 and bw.gy.cols.inv.size == 16
    assert fw.w.cols.inv.size == 32 and fw.x.cols.inv.size == 32
