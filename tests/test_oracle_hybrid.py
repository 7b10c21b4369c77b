"""Pins of the oracle's row-split hybrid GEMM ("Production 2:4 Structured
Sparsity for LLMs", section "Dense Fallback and Hybrid Sparsity Design"):
with one region empty it is the plain sparse or the plain dense product, its
column blocks are those products, a dense region holding pruned rows gives
what the compressed rows give, and permuting the weight rows permutes the
output columns."""
import numpy as np

import oracle
from semi_structured_sparse_sp24_amd import inputs


def _ops(dt, M, NS, ND, K, seed):
    x = inputs.to_bits(inputs.normal((M, K), 1.0, seed), dt)
    ws = inputs.to_bits(inputs.normal((NS, K), 0.5, seed + 1), dt)
    wd = inputs.to_bits(inputs.normal((ND, K), 0.5, seed + 2), dt)
    v, m = oracle.prune_compress(dt, ws)
    return x, ws, v, m, wd


def test_empty_regions_reduce_to_the_plain_products():
    dt = oracle.BF16
    x, ws, v, m, wd = _ops(dt, 5, 16, 24, 64, 3)
    R = oracle.hybrid_gemm(dt, 5, 16, 0, 64, x=x, ws_vals=v, ws_meta=m)
    assert np.array_equal(R, oracle.gemm(dt, 5, 16, 64, x=x, w_vals=v, w_meta=m))
    R = oracle.hybrid_gemm(dt, 5, 0, 24, 64, x=x, wd=wd)
    assert np.array_equal(R, oracle.gemm(dt, 5, 24, 64, x=x, w=wd))


def test_pruned_rows_in_the_dense_region_match_the_compressed_ones():
    dt = oracle.F16
    x, ws, v, m, _ = _ops(dt, 7, 8, 0, 128, 9)
    pruned = oracle.decompress(dt, v, m, 128)
    R = oracle.hybrid_gemm(dt, 7, 8, 8, 128, x=x, ws_vals=v, ws_meta=m, wd=pruned)
    assert np.array_equal(R[:, :8], R[:, 8:])
    # and against numpy on the decoded operands
    X, P = oracle.decode(dt, x), oracle.decode(dt, pruned)
    assert np.allclose(R[:, :8], X @ P.T, rtol=1e-12, atol=1e-12)


def test_row_permutation_permutes_columns_and_scales_apply_per_column():
    dt = oracle.E4M3
    M, NS, ND, K = 4, 8, 6, 128
    x = inputs.quantize_e4m3_rows(inputs.normal((M, K), 1.0, 1))[0]
    ws = inputs.quantize_e4m3_rows(inputs.normal((NS, K), 1.0, 2))[0]
    wd = inputs.quantize_e4m3_rows(inputs.normal((ND, K), 1.0, 3))[0]
    v, m = oracle.prune_compress(dt, ws)
    sx = np.linspace(0.5, 2.0, M).astype(np.float32)
    sw = np.linspace(0.25, 4.0, NS + ND).astype(np.float32)
    R = oracle.hybrid_gemm(dt, M, NS, ND, K, x=x, ws_vals=v, ws_meta=m, wd=wd, scale_x=sx, scale_w=sw)
    U = oracle.hybrid_gemm(dt, M, NS, ND, K, x=x, ws_vals=v, ws_meta=m, wd=wd)
    assert np.allclose(R, U * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64), rtol=1e-12)
    p = np.random.default_rng(0).permutation(ND)
    Rp = oracle.hybrid_gemm(dt, M, NS, ND, K, x=x, ws_vals=v, ws_meta=m, wd=wd[p])
    assert np.array_equal(Rp[:, NS:], U[:, NS:][:, p])
