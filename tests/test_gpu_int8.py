"""GPU parity of the 2:4 + INT8 path (two's complement int8 operands, |x|
magnitude, int32 accumulation, per-row fp32 scales; the 2:4-versus-
quantization paper, section 4.2 "Speed"): prune+compress and decompress
byte-exact against the oracle, every GEMM kernel (decode, tile, dense,
hybrid) against the oracle's product, and bitwise on small integers with
fp32 output."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, decode_out, say, to_dev, to_host, meta_host

pytestmark = pytest.mark.gpu
I8 = oracle.I8


def _ints(shape, seed, lo=-128, hi=127):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.int8).view(np.uint8)


@pytest.mark.parametrize("rows,K", [(3, 128), (37, 1024), (5, 36), (130, 4112)])
def test_prune_compress_and_decompress_bytewise(rows, K):
    say("int8 compress", rows, K)
    bits = _ints((rows, K), rows + K)
    bits[0, :8] = np.array([-128, 127, -127, 1, -1, 1, -1, 1], dtype=np.int8).view(np.uint8)
    v, m = oracle.prune_compress(I8, bits)
    gv, gm = sp.prune_compress(to_dev(bits, I8))
    back = sp.decompress(gv, gm, K)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(gv, I8), v)
    assert np.array_equal(meta_host(gm), m)
    assert np.array_equal(to_host(back, I8), oracle.decompress(I8, v, m, K))


# decode kernels (M <= 64, with 32-row tiles on the wide ones), tile kernels (M = 512; larger M on
# sampled rows), including the 128x128 tiles and the quarter-tile tail of a 320-tile grid
GEMM = [(1, 4096, 1024), (4, 1000, 512), (8, 8192, 512), (16, 2048, 1024), (24, 1024, 512), (33, 640, 512),
        (64, 768, 2048), (512, 1536, 1024), (4096, 2048, 512), (2048, 6144, 256),
        (24, 6150, 512), (48, 5200, 512), (1024, 3072, 512), (4096, 5120, 512)]


def _operands(M, N, K, seed):
    xb, sx = inputs.quantize_i8_rows(inputs.normal((M, K), 1.0, seed))
    wb, sw = inputs.quantize_i8_rows(inputs.normal((N, K), 0.02, seed + 1))
    return xb, sx, wb, sw


@pytest.mark.parametrize("M,N,K", GEMM)
def test_sparse_w_and_dense_match_oracle(M, N, K):
    xb, sx, wb, sw = _operands(M, N, K, M + N)
    v, m = oracle.prune_compress(I8, wb)
    X, V, Mt = to_dev(xb, I8), to_dev(v, I8), torch.from_numpy(m.view(np.int32)).cuda()
    Wp = to_dev(oracle.decompress(I8, v, m, K), I8)
    tsx, tsw = torch.from_numpy(sx).cuda(), torch.from_numpy(sw).cuda()
    say("int8 gemm", M, N, K, sp.gemm_kernel(True, sp.SPARSE_W, torch.int8, torch.bfloat16, M, N, K),
        sp.gemm_kernel(False, sp.SPARSE_W, torch.int8, torch.bfloat16, M, N, K))
    Y = sp.sp24_gemm(sp.SPARSE_W, V, Mt, X, M, N, K, scale_x=tsx, scale_w=tsw)
    Yd = sp.dense_gemm(X, Wp, scale_x=tsx, scale_w=tsw)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 512 else np.unique(np.r_[0, M - 1, np.random.default_rng(1).integers(0, M, 40)])
    R = oracle.gemm(I8, M, N, K, x=xb, w_vals=v, w_meta=m, scale_x=sx, scale_w=sw, mrows=rows)
    assert oracle.relative_error(decode_out(Y)[rows], R) <= TOL[I8]
    assert oracle.relative_error(decode_out(Yd)[rows], R) <= TOL[I8]


@pytest.mark.parametrize("M,N,K", [(4, 512, 1024), (48, 640, 512), (300, 520, 1024), (1024, 2048, 512)])
def test_small_integers_are_exact(M, N, K):
    """|x|, |w| <= 16: every int32 partial sum and its fp32 conversion are
    exact, so the sparse and dense kernels match the oracle bit for bit."""
    xb, wb = _ints((M, K), 5 + M, -16, 16), _ints((N, K), 6 + N, -16, 16)
    v, m = oracle.prune_compress(I8, wb)
    X, V, Mt = to_dev(xb, I8), to_dev(v, I8), torch.from_numpy(m.view(np.int32)).cuda()
    Wp = to_dev(oracle.decompress(I8, v, m, K), I8)
    say("int8 exact", M, N, K)
    Y = sp.sp24_gemm(sp.SPARSE_W, V, Mt, X, M, N, K, out_dtype=torch.float32)
    Yd = sp.dense_gemm(X, Wp, out_dtype=torch.float32)
    xv, xm = oracle.prune_compress(I8, xb)
    Yx = sp.sp24_gemm(sp.SPARSE_X, to_dev(xv, I8), torch.from_numpy(xm.view(np.int32)).cuda(), to_dev(wb, I8),
                      M, N, K, out_dtype=torch.float32)
    torch.cuda.synchronize()
    R = oracle.gemm(I8, M, N, K, x=xb, w_vals=v, w_meta=m)
    assert np.array_equal(decode_out(Y), R)
    assert np.array_equal(decode_out(Yd), R)
    assert np.array_equal(decode_out(Yx), oracle.gemm(I8, M, N, K, x_vals=xv, x_meta=xm, w=wb))


def test_hybrid_int8():
    M, NS, ND, K = 256, 512, 264, 1024
    xb, sx, wb, sw = _operands(M, NS + ND, K, 77)
    v, m = oracle.prune_compress(I8, wb[:NS])
    say("int8 hybrid", M, NS, ND, K)
    Y = sp.hybrid_gemm(to_dev(v, I8), torch.from_numpy(m.view(np.int32)).cuda(), to_dev(wb[NS:], I8),
                       to_dev(xb, I8), NS, ND, scale_x=torch.from_numpy(sx).cuda(),
                       scale_w=torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    R = oracle.hybrid_gemm(I8, M, NS, ND, K, x=xb, ws_vals=v, ws_meta=m, wd=wb[NS:], scale_x=sx, scale_w=sw)
    assert oracle.relative_error(decode_out(Y), R) <= TOL[I8]
