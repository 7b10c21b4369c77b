"""Pins of the oracle's K-split hybrid product (columns [0, KS) of every
weight row 2:4, columns [KS, K) dense; "Production 2:4 Structured Sparsity
for LLMs", "Dense Fallback and Hybrid Sparsity Design", and the Spense
abstract on the SlideSparse page).  Each pin is something the definition
fixes independently of how the oracle computes it:

  - the two degenerate splits are the plain 2:4 product and the plain dense
    product;
  - one-hot rows of X read back single weight entries: the pruned 2:4 value
    in the first range and the dense value in the second, at the right
    column (numbers taken from the inputs, not from a product);
  - the product is the sum of the two ranges' products over the matching
    columns of X (an offset of the dense range, or a dropped range, breaks it);
  - scales multiply the whole sum.
Planted mistakes (wrong offset, dropped range, swapped ranges, scales on one
range only) each fail at least one pin."""
import numpy as np
import pytest
import torch

import oracle
from semi_structured_sparse_sp24_amd import inputs


def _ints(shape, seed, lo=-3, hi=3):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def _bits(a, dt):
    """Small integers (exact in every format) as bit patterns of format dt."""
    if dt == oracle.I8:
        return a.astype(np.int8).view(np.uint8)
    return inputs.to_bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)), dt)


def _operands(dt, M, N, KS, K, seed, integer=True):
    KD = K - KS
    if integer or dt == oracle.I8:
        x = _bits(_ints((M, K), seed), dt)
        w = _bits(_ints((N, K), seed + 1), dt)
    else:
        x = inputs.to_bits(inputs.normal((M, K), 1.0, seed), dt)
        w = inputs.to_bits(inputs.normal((N, K), 0.02, seed + 1), dt)
    ws = np.ascontiguousarray(w[:, :KS])
    wd = np.ascontiguousarray(w[:, KS:])
    v, m = oracle.prune_compress(dt, ws) if KS else (np.zeros((N, 0), w.dtype), np.zeros((N, 0), np.uint32))
    assert wd.shape == (N, KD)
    return x, w, ws, wd, v, m


def _ksplit(dt, M, N, KS, K, x, v, m, wd, **kw):
    return oracle.ksplit_gemm(dt, M, N, KS, K, x=x, ws_vals=v, ws_meta=m, wd=wd, **kw)


# planted mistakes: each is the K-split product computed wrongly in one way
def _wrong_offset(dt, M, N, KS, K, x, v, m, wd, **kw):
    """The dense range multiplied by the first KD columns of X."""
    KD = K - KS
    xs = np.ascontiguousarray(x[:, :KS])
    xd = np.ascontiguousarray(x[:, :KD])
    return oracle.gemm(dt, M, N, KS, x=xs, w_vals=v, w_meta=m) + oracle.gemm(dt, M, N, KD, x=xd, w=wd)


def _dropped_dense(dt, M, N, KS, K, x, v, m, wd, **kw):
    return oracle.gemm(dt, M, N, KS, x=np.ascontiguousarray(x[:, :KS]), w_vals=v, w_meta=m)


def _swapped(dt, M, N, KS, K, x, v, m, wd, **kw):
    """The dense range placed first along K."""
    w = np.concatenate([wd, oracle.decompress(dt, v, m, KS)], axis=1)
    return oracle.gemm(dt, M, N, K, x=x, w=np.ascontiguousarray(w))


def _scale_sparse_only(dt, M, N, KS, K, x, v, m, wd, scale_x=None, scale_w=None):
    xs, xd = np.ascontiguousarray(x[:, :KS]), np.ascontiguousarray(x[:, KS:])
    return oracle.gemm(dt, M, N, KS, x=xs, w_vals=v, w_meta=m, scale_x=scale_x, scale_w=scale_w) + \
        oracle.gemm(dt, M, N, K - KS, x=xd, w=wd)


IMPLS = {"oracle": _ksplit, "wrong_offset": _wrong_offset, "dropped_dense": _dropped_dense,
         "swapped": _swapped, "scale_sparse_only": _scale_sparse_only}


def _pins(impl, dt=oracle.BF16):
    """Runs every pin on `impl`; returns the names of the pins it fails."""
    failed = []
    M, N, KS, K = 6, 10, 32, 48
    x, w, ws, wd, v, m = _operands(dt, M, N, KS, K, 11)
    # degenerate splits
    R = impl(dt, M, N, K, K, x, *oracle.prune_compress(dt, w), np.zeros((N, 0), w.dtype))
    if not np.array_equal(R, oracle.gemm(dt, M, N, K, x=x, w=oracle.prune(dt, w))):
        failed.append("all 2:4")
    R = impl(dt, M, N, 0, K, x, np.zeros((N, 0), w.dtype), np.zeros((N, 0), np.uint32), w)
    if not np.array_equal(R, oracle.gemm(dt, M, N, K, x=x, w=w)):
        failed.append("all dense")
    # one-hot rows of X read single entries of the assembled weight
    eye = np.zeros((K, K), dtype=np.float32)
    eye[np.arange(K), np.arange(K)] = 1.0
    xe = _bits(eye, dt)
    R = impl(dt, K, N, KS, K, xe, v, m, wd)
    pruned = oracle.decode(dt, oracle.prune(dt, ws))
    dense = oracle.decode(dt, wd)
    if not (np.array_equal(R[:KS], pruned.T) and np.array_equal(R[KS:], dense.T)):
        failed.append("one-hot")
    # the sum of the ranges' products over the matching columns of X
    xn, _, _, wdn, vn, mn = _operands(dt, M, N, KS, K, 12, integer=False)
    R = impl(dt, M, N, KS, K, xn, vn, mn, wdn)
    parts = oracle.gemm(dt, M, N, KS, x=np.ascontiguousarray(xn[:, :KS]), w_vals=vn, w_meta=mn) + \
        oracle.gemm(dt, M, N, K - KS, x=np.ascontiguousarray(xn[:, KS:]), w=wdn)
    if not np.allclose(R, parts, rtol=1e-12, atol=1e-12):
        failed.append("sum of ranges")
    # scales multiply the whole sum: on integers, power-of-two scales keep everything exact
    sx = (2.0 ** np.arange(M) / 8).astype(np.float32)
    sw = (2.0 ** -np.arange(N)).astype(np.float32)
    R = impl(dt, M, N, KS, K, x, v, m, wd, scale_x=sx, scale_w=sw)
    R0 = impl(dt, M, N, KS, K, x, v, m, wd)
    if not np.array_equal(R, R0 * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64)):
        failed.append("scales")
    return failed


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3, oracle.I8])
def test_oracle_meets_every_pin(dt):
    assert _pins(_ksplit, dt) == []


@pytest.mark.parametrize("name", [n for n in IMPLS if n != "oracle"])
def test_planted_mistakes_fail_a_pin(name):
    assert _pins(IMPLS[name]) != [], name


def test_bench_split_is_whole_blocks():
    """The bench's split keeps the 2:4 range in whole 256-column blocks (the
    GEMM's metadata blocks) and a dense quarter of K."""
    for N, K in inputs.WORKLOADS["ksplit"]["shapes"]:
        KS, KD = inputs.ksplit_split(K)
        assert KS + KD == K and KS % 256 == 0 and KD % 256 == 0 and KD == K // 4
