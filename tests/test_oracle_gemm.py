"""Pins the oracle GEMM: against float64 matmul on the decompressed operand
(a library routine), exact integer products, one-hot rows that read back the
decompressed weight rows (metadata addressing), scale application and row
subsets."""
import numpy as np
import pytest
import torch

import oracle
from semi_structured_sparse_sp24_amd import inputs


def _f64(dt, bits):
    """Decode through torch, independently of the oracle's own codecs."""
    if dt == oracle.E4M3:
        return torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64)
    tdt = torch.float16 if dt == oracle.F16 else torch.bfloat16
    return torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float64)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16, oracle.E4M3])
def test_sparse_w_matches_float64_matmul(dt):
    M, N, K = 9, 40, 192
    w = inputs.normal((N, K), 0.5, 1)
    x = inputs.normal((M, K), 1.0, 2)
    if dt == oracle.E4M3:
        wb, sw = inputs.quantize_e4m3_rows(w)
        xb, sx = inputs.quantize_e4m3_rows(x)
    else:
        wb, sw, xb, sx = inputs.to_bits(w, dt), None, inputs.to_bits(x, dt), None
    wv, wm = oracle.prune_compress(dt, wb)
    R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw)
    wp = oracle.decompress(dt, wv, wm, K)
    ref = _f64(dt, xb) @ _f64(dt, wp).T
    if sx is not None:
        ref = ref * torch.from_numpy(sx).double()[:, None] * torch.from_numpy(sw).double()[None, :]
    np.testing.assert_allclose(R, ref.numpy(), rtol=1e-12, atol=1e-12 * float(ref.abs().max()))


def test_sparse_x_matches_float64_matmul():
    dt, M, N, K = oracle.BF16, 24, 16, 128
    xb = inputs.to_bits(inputs.normal((M, K), 1.0, 3), dt)
    wb = inputs.to_bits(inputs.normal((N, K), 0.02, 4), dt)
    xv, xm = oracle.prune_compress(dt, xb)
    R = oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb)
    ref = _f64(dt, oracle.decompress(dt, xv, xm, K)) @ _f64(dt, wb).T
    np.testing.assert_allclose(R, ref.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16, oracle.E4M3])
def test_exact_integer_product(dt):
    """Entries in -3..3: every sum is an integer the int64 product gives exactly."""
    M, N, K = 17, 33, 512
    xb = inputs.integer_operand((M, K), 5, dt)
    wb = inputs.integer_operand((N, K), 6, dt)
    wv, wm = oracle.prune_compress(dt, wb)
    R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm)
    xi = _f64(dt, xb).numpy().astype(np.int64)
    wpi = _f64(dt, oracle.decompress(dt, wv, wm, K)).numpy().astype(np.int64)
    assert np.array_equal(R, (xi @ wpi.T).astype(np.float64))
    # the dense path on the same pruned operand is the same product
    R2 = oracle.gemm(dt, M, N, K, x=xb, w=oracle.decompress(dt, wv, wm, K))
    assert np.array_equal(R, R2)


def test_one_hot_rows_read_back_decompressed_weights():
    """X = rows of the identity: Y[m, n] = Wp[n, m], which exercises every
    metadata position and word."""
    dt, N, K = oracle.BF16, 48, 96
    wb = inputs.to_bits(inputs.normal((N, K), 1.0, 7), dt)
    wv, wm = oracle.prune_compress(dt, wb)
    x = inputs.to_bits(torch.eye(K), dt)
    R = oracle.gemm(dt, K, N, K, x=x, w_vals=wv, w_meta=wm)
    wp = oracle.decode(dt, oracle.decompress(dt, wv, wm, K))
    assert np.array_equal(R, wp.T)


def test_row_subset_matches_full():
    dt, M, N, K = oracle.F16, 20, 12, 64
    xb = inputs.to_bits(inputs.normal((M, K), 1.0, 8), dt)
    wb = inputs.to_bits(inputs.normal((N, K), 0.02, 9), dt)
    wv, wm = oracle.prune_compress(dt, wb)
    full = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm)
    rows = np.array([19, 0, 7, 7])
    sub = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, mrows=rows)
    assert np.array_equal(sub, full[rows])


def test_scales_multiply_rows_and_columns():
    dt, M, N, K = oracle.E4M3, 6, 10, 128
    xb = inputs.integer_operand((M, K), 10, dt)
    wb = inputs.integer_operand((N, K), 11, dt)
    sx = np.linspace(0.5, 3.0, M).astype(np.float32)
    sw = np.linspace(-2.0, 1.0, N).astype(np.float32)
    wv, wm = oracle.prune_compress(dt, wb)
    plain = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm)
    scaled = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw)
    expect = plain * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    np.testing.assert_allclose(scaled, expect, rtol=1e-15)


def test_relative_error_measure():
    R = np.array([[1.0, -2.0], [0.0, 4.0]])
    assert oracle.relative_error(R, R) == 0.0
    rms = np.sqrt(np.mean(R * R))
    Y = R.copy()
    Y[1, 0] = 0.1                               # near-zero output: floored at rms
    assert oracle.relative_error(Y, R) == pytest.approx(0.1 / rms)
    Y = R * (1 + 1e-3)
    assert oracle.relative_error(Y, R) == pytest.approx(1e-3)
