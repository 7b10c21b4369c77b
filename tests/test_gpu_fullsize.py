"""Full-size parity of the bench workloads that combine several kernels:

  - online_fp8: the bf16 activation (4096 x 4096, 1% outliers x20) through
    the fused quantize + prune + compress (codes, metadata and scales byte
    for byte against the oracle), then the scaled fp8 activation-compressed
    GEMM against both weight shapes; and the dense side, the plain quantizer
    and the dense fp8 GEMM on its codes;
  - online_int8: the same activation through the fused int8 quantize +
    prune + compress (byte for byte), then the int8 activation-compressed
    GEMM against both weight shapes, and the dense side on the plain codes;
  - int8: every (shape, M) case, weight-compressed GEMM and the dense GEMM
    on the decompressed weight, with per-row scales (K up to 25600);
  - hybrid: every (shape, M) case of the row-split hybrid GEMM.

Each case runs at the bench's shapes, so the dispatcher picks the kernels
the bench times, and compares one row from every 256-row band of M (plus the
first and last rows) with the oracle's fp64 product; every output must be
finite."""
import functools

import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, band_rows, decode_out, meta_host, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _cases(wl):
    w = inputs.WORKLOADS[wl]
    return [(s, j) for s in range(len(w["shapes"])) for j in range(len(w["ms"]))]


def _f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@functools.lru_cache(maxsize=1)
def _weight(wl, s):
    return inputs.weight(wl, s)


@functools.lru_cache(maxsize=1)
def _online_fp8_x(s):
    """The online fp8 activation of weight shape s (as the bench draws it), and
    the oracle's fused and plain quantizations of it."""
    xb, _ = inputs.activation("online_fp8", s, 0)
    xv, xm, xs = oracle.quantize_prune_compress(oracle.BF16, xb)
    xq, xqs = oracle.quantize_e4m3_rows(oracle.BF16, xb)
    return xb, xv, xm, xs, xq, xqs


@pytest.mark.parametrize("s", range(len(inputs.WORKLOADS["online_fp8"]["shapes"])))
def test_online_fp8_end_to_end(s):
    w = inputs.WORKLOADS["online_fp8"]
    N, K = w["shapes"][s]
    M = w["ms"][0]
    name = sp.gemm_kernel(True, sp.SPARSE_X, torch.float8_e4m3fn, torch.bfloat16, M, N, K)
    say("full online_fp8", (N, K), "M", M, name)
    xb, xv, xm, xs, xq, xqs = _online_fp8_x(s)
    wb, sw = _weight("online_fp8", s)
    X = to_dev(xb, oracle.BF16)
    W = to_dev(wb, oracle.E4M3)
    gv, gm, gs = sp.quantize_prune_compress(X)
    gq, gqs = sp.quantize_e4m3(X)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(gv, oracle.E4M3), xv)
    assert np.array_equal(meta_host(gm), xm)
    assert np.array_equal(gs.cpu().numpy(), xs)
    assert np.array_equal(to_host(gq, oracle.E4M3), xq)
    assert np.array_equal(gqs.cpu().numpy(), xqs)
    Y = sp.sp24_gemm(sp.SPARSE_X, gv, gm, W, M, N, K, scale_x=gs, scale_w=_f32(sw))
    Yd = sp.dense_gemm(gq, W, scale_x=gqs, scale_w=_f32(sw))
    torch.cuda.synchronize()
    rows = band_rows(M, seed=s)
    R = oracle.gemm(oracle.E4M3, M, N, K, x_vals=xv, x_meta=xm, w=wb, scale_x=xs, scale_w=sw, mrows=rows)
    Rd = oracle.gemm(oracle.E4M3, M, N, K, x=xq, w=wb, scale_x=xqs, scale_w=sw, mrows=rows)
    rt = torch.from_numpy(rows).cuda()
    e_s, e_d = oracle.relative_error(decode_out(Y[rt]), R), oracle.relative_error(decode_out(Yd[rt]), Rd)
    say("  rel err sparse", e_s, "dense", e_d)
    assert e_s <= TOL[oracle.E4M3] and e_d <= TOL[oracle.E4M3]
    assert bool(torch.isfinite(Y.float()).all()) and bool(torch.isfinite(Yd.float()).all())


@functools.lru_cache(maxsize=1)
def _online_int8_x(s):
    xb, _ = inputs.activation("online_int8", s, 0)
    xv, xm, xs = oracle.quantize_i8_prune_compress(oracle.BF16, xb)
    xq, xqs = oracle.quantize_i8_rows(oracle.BF16, xb)
    return xb, xv, xm, xs, xq, xqs


@pytest.mark.parametrize("s", range(len(inputs.WORKLOADS["online_int8"]["shapes"])))
def test_online_int8_end_to_end(s):
    w = inputs.WORKLOADS["online_int8"]
    N, K = w["shapes"][s]
    M = w["ms"][0]
    name = sp.gemm_kernel(True, sp.SPARSE_X, torch.int8, torch.bfloat16, M, N, K)
    say("full online_int8", (N, K), "M", M, name)
    xb, xv, xm, xs, xq, xqs = _online_int8_x(s)
    wb, sw = _weight("online_int8", s)
    X = to_dev(xb, oracle.BF16)
    W = to_dev(wb, oracle.I8)
    gv, gm, gs = sp.quantize_i8_prune_compress(X)
    gq, gqs = sp.quantize_i8(X)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(gv, oracle.I8), xv)
    assert np.array_equal(meta_host(gm), xm)
    assert np.array_equal(gs.cpu().numpy(), xs)
    assert np.array_equal(to_host(gq, oracle.I8), xq)
    assert np.array_equal(gqs.cpu().numpy(), xqs)
    Y = sp.sp24_gemm(sp.SPARSE_X, gv, gm, W, M, N, K, scale_x=gs, scale_w=_f32(sw))
    Yd = sp.dense_gemm(gq, W, scale_x=gqs, scale_w=_f32(sw))
    torch.cuda.synchronize()
    rows = band_rows(M, seed=s + 7)
    R = oracle.gemm(oracle.I8, M, N, K, x_vals=xv, x_meta=xm, w=wb, scale_x=xs, scale_w=sw, mrows=rows)
    Rd = oracle.gemm(oracle.I8, M, N, K, x=xq, w=wb, scale_x=xqs, scale_w=sw, mrows=rows)
    rt = torch.from_numpy(rows).cuda()
    e_s, e_d = oracle.relative_error(decode_out(Y[rt]), R), oracle.relative_error(decode_out(Yd[rt]), Rd)
    say("  rel err sparse", e_s, "dense", e_d)
    assert e_s <= TOL[oracle.I8] and e_d <= TOL[oracle.I8]
    assert bool(torch.isfinite(Y.float()).all()) and bool(torch.isfinite(Yd.float()).all())


@functools.lru_cache(maxsize=1)
def _int8_weight(s):
    wb, sw = inputs.weight("int8", s)
    wv, wm = oracle.prune_compress(oracle.I8, wb)
    return wb, sw, wv, wm


@pytest.mark.parametrize("s,j", _cases("int8"))
def test_int8_full_size(s, j):
    w = inputs.WORKLOADS["int8"]
    N, K = w["shapes"][s]
    M = w["ms"][j]
    name = sp.gemm_kernel(True, sp.SPARSE_W, torch.int8, torch.bfloat16, M, N, K)
    say("full int8", (N, K), "M", M, name)
    wb, sw, wv, wm = _int8_weight(s)
    xb, sx = inputs.activation("int8", s, j)
    W, X = to_dev(wb, oracle.I8), to_dev(xb, oracle.I8)
    v, m = sp.prune_compress(W)
    Wp = sp.decompress(v, m, K)
    Y = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, scale_x=_f32(sx), scale_w=_f32(sw))
    Yd = sp.dense_gemm(X, Wp, scale_x=_f32(sx), scale_w=_f32(sw))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(v, oracle.I8), wv) and np.array_equal(meta_host(m), wm)
    rows = band_rows(M, seed=10 * s + j)
    R = oracle.gemm(oracle.I8, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw, mrows=rows)
    rt = torch.from_numpy(rows).cuda()
    e_s, e_d = oracle.relative_error(decode_out(Y[rt]), R), oracle.relative_error(decode_out(Yd[rt]), R)
    say("  rel err sparse", e_s, "dense", e_d)
    assert e_s <= TOL[oracle.I8] and e_d <= TOL[oracle.I8]
    assert bool(torch.isfinite(Y.float()).all()) and bool(torch.isfinite(Yd.float()).all())


@functools.lru_cache(maxsize=1)
def _hybrid_weight(s):
    N, _ = inputs.WORKLOADS["hybrid"]["shapes"][s]
    NS, ND = inputs.hybrid_split(N)
    wb, _ = inputs.weight("hybrid", s)
    wv, wm = oracle.prune_compress(oracle.BF16, wb[:NS])
    return wb, NS, ND, wv, wm


@pytest.mark.parametrize("s,j", _cases("hybrid"))
def test_hybrid_full_size(s, j):
    w = inputs.WORKLOADS["hybrid"]
    N, K = w["shapes"][s]
    M = w["ms"][j]
    wb, NS, ND, wv, wm = _hybrid_weight(s)
    name = sp.hybrid_kernel(torch.bfloat16, torch.bfloat16, M, NS, ND, K)
    say("full hybrid", (N, K), NS, "+", ND, "M", M, name)
    xb, _ = inputs.activation("hybrid", s, j)
    W, X = to_dev(wb, oracle.BF16), to_dev(xb, oracle.BF16)
    v, m = sp.prune_compress(W[:NS].contiguous())
    Y = sp.hybrid_gemm(v, m, W[NS:].contiguous(), X, NS, ND)
    torch.cuda.synchronize()
    rows = band_rows(M, seed=10 * s + j)
    R = oracle.hybrid_gemm(oracle.BF16, len(rows), NS, ND, K, x=xb[rows], ws_vals=wv, ws_meta=wm, wd=wb[NS:])
    rt = torch.from_numpy(rows).cuda()
    Yr = decode_out(Y[rt])
    e_s = oracle.relative_error(Yr[:, :NS], R[:, :NS])
    e_d = oracle.relative_error(Yr[:, NS:], R[:, NS:])
    say("  rel err 2:4 rows", e_s, "dense rows", e_d)
    assert e_s <= TOL[oracle.BF16] and e_d <= TOL[oracle.BF16]
    assert bool(torch.isfinite(Y.float()).all())
