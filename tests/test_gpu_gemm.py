"""GPU parity of the sparse GEMM (weight- and activation-sparse) and the
dense GEMM against the oracle's fp64 product on the decompressed operand:

  - small shapes spanning several tiles with ragged tails, both kernel
    families (skinny M <= 64 and tiled), every dtype and output type;
  - exact-integer inputs, where fp32 accumulation is exact and the GPU output
    must equal the oracle bit for bit;
  - every workload at full size in the launch configuration the bench uses,
    checked on sampled rows of M;
  - edge cases: empty outputs, K = 0, ineligible K, guard bands, reruns.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, band_rows, decode_out, say, to_dev, to_host

pytestmark = pytest.mark.gpu

OUT_T = {oracle.F16: torch.float16, oracle.BF16: torch.bfloat16, oracle.F32: torch.float32}


def _operands(dt, M, N, K, seed, integer=False):
    if integer:
        xb = inputs.integer_operand((M, K), seed, dt)
        wb = inputs.integer_operand((N, K), seed + 1, dt)
        return xb, None, wb, None
    x = inputs.normal((M, K), 1.0, seed)
    w = inputs.normal((N, K), 0.02, seed + 1)
    if dt == oracle.E4M3:
        xb, sx = inputs.quantize_e4m3_rows(x)
        wb, sw = inputs.quantize_e4m3_rows(w)
        return xb, sx, wb, sw
    return inputs.to_bits(x, dt), None, inputs.to_bits(w, dt), None


def _sparse_w(dt, out, M, N, K, seed=1, integer=False, mrows=None):
    xb, sx, wb, sw = _operands(dt, M, N, K, seed, integer)
    wv, wm = oracle.prune_compress(dt, wb)
    R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw, mrows=mrows)
    W = to_dev(wb, dt)
    X = to_dev(xb, dt)
    v, m = sp.prune_compress(W)
    dsx = None if sx is None else torch.from_numpy(sx).cuda()
    dsw = None if sw is None else torch.from_numpy(sw).cuda()
    Y = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out_dtype=OUT_T[out], scale_x=dsx, scale_w=dsw)
    torch.cuda.synchronize()
    Yh = decode_out(Y)
    return (Yh if mrows is None else Yh[mrows]), R, Y


def _sparse_x(dt, out, M, N, K, seed=1, integer=False):
    xb, sx, wb, sw = _operands(dt, M, N, K, seed, integer)
    xv, xm = oracle.prune_compress(dt, xb)
    R = oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, scale_x=sx, scale_w=sw)
    v, m = sp.prune_compress(to_dev(xb, dt))
    dsx = None if sx is None else torch.from_numpy(sx).cuda()
    dsw = None if sw is None else torch.from_numpy(sw).cuda()
    Y = sp.sp24_gemm(sp.SPARSE_X, v, m, to_dev(wb, dt), M, N, K, out_dtype=OUT_T[out],
                     scale_x=dsx, scale_w=dsw)
    torch.cuda.synchronize()
    return decode_out(Y), R, Y


def _dense(dt, out, M, N, K, seed=1, integer=False, prune_w=True):
    xb, sx, wb, sw = _operands(dt, M, N, K, seed, integer)
    if prune_w:
        wb = oracle.prune(dt, wb)
    R = oracle.gemm(dt, M, N, K, x=xb, w=wb, scale_x=sx, scale_w=sw)
    dsx = None if sx is None else torch.from_numpy(sx).cuda()
    dsw = None if sw is None else torch.from_numpy(sw).cuda()
    Y = sp.dense_gemm(to_dev(xb, dt), to_dev(wb, dt), out_dtype=OUT_T[out], scale_x=dsx, scale_w=dsw)
    torch.cuda.synchronize()
    return decode_out(Y), R, Y


DT_OUT = [(oracle.BF16, oracle.BF16), (oracle.F16, oracle.F16), (oracle.BF16, oracle.F32),
          (oracle.F16, oracle.BF16), (oracle.E4M3, oracle.BF16), (oracle.E4M3, oracle.F32)]
SMALL = [(1, 16, 256), (4, 48, 256), (16, 130, 512), (17, 33, 256), (63, 64, 384), (64, 200, 256),
         (65, 130, 256), (200, 96, 512), (300, 260, 1024)]


def _k(dt, K):
    return K if dt != oracle.E4M3 else max(128, K // 128 * 128)


@pytest.mark.parametrize("dt,out", DT_OUT)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_sparse_w_small(dt, out, M, N, K):
    K = _k(dt, K)
    say("sparse_w", dt, out, M, N, K)
    Y, R, _ = _sparse_w(dt, out, M, N, K, seed=M * 31 + N)
    assert oracle.relative_error(Y, R) <= TOL[dt]


@pytest.mark.parametrize("dt,out", DT_OUT)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_sparse_x_small(dt, out, M, N, K):
    K = _k(dt, K)
    say("sparse_x", dt, out, M, N, K)
    Y, R, _ = _sparse_x(dt, out, M, N, K, seed=M * 37 + N)
    assert oracle.relative_error(Y, R) <= TOL[dt]


@pytest.mark.parametrize("dt,out", DT_OUT)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_dense_small(dt, out, M, N, K):
    K = _k(dt, K)
    say("dense", dt, out, M, N, K)
    Y, R, _ = _dense(dt, out, M, N, K, seed=M * 41 + N)
    assert oracle.relative_error(Y, R) <= TOL[dt]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3])
@pytest.mark.parametrize("M,N,K", [(1, 64, 1024), (16, 48, 2048), (64, 128, 512), (130, 200, 1024),
                                   (256, 256, 2048)])
def test_exact_integer_bitwise(dt, M, N, K):
    """|sums| < 2^24: fp32 accumulation is exact in any order, so f32 output
    equals the oracle exactly and 16-bit output equals its RNE encoding."""
    K = _k(dt, K)
    say("exact", dt, M, N, K)
    Y, R, _ = _sparse_w(dt, oracle.F32, M, N, K, seed=M + N, integer=True)
    assert np.array_equal(Y, R)
    Y, R, _ = _sparse_x(dt, oracle.F32, M, N, K, seed=M + N + 5, integer=True)
    assert np.array_equal(Y, R)
    Y, R, _ = _dense(dt, oracle.F32, M, N, K, seed=M + N + 9, integer=True)
    assert np.array_equal(Y, R)
    Y, R, Yd = _sparse_w(dt, oracle.BF16, M, N, K, seed=M + N + 13, integer=True)
    assert np.array_equal(to_host(Yd, oracle.BF16), oracle.encode(oracle.BF16, R))
    if dt != oracle.E4M3:
        Y, R, Yd = _sparse_x(dt, oracle.F16, M, N, K, seed=M + N + 17, integer=True)
        assert np.array_equal(to_host(Yd, oracle.F16), oracle.encode(oracle.F16, R))


# one case per decode kernel variant: ragged rows of A (not a multiple of the
# 16- or 32-row tile) and a partial last group of 8 K steps
SKINNY = [(1, 100, 704, "sp24_skinny_x4"), (4, 6150, 704, "sp24_skinny_x4"),
          (9, 300, 704, "sp24_skinny_m16"), (16, 6150, 704, "sp24_skinny_m16_a32"),
          (7, 6166, 1216, "sp24_skinny_m16_a32"), (30, 200, 704, "sp24_skinny_m32"),
          (64, 190, 704, "sp24_skinny_m64"), (50, 333, 192, "sp24_skinny_m64"),
          (40, 17000, 704, "sp24_big_128x64"), (17, 61500, 192, "sp24_big_256x64"),
          # 32-row A tiles for 17 to 64 rows once there are 160 or more of them
          (30, 6150, 704, "sp24_skinny_m32_a32"), (64, 5200, 704, "sp24_skinny_m64_a32"),
          (50, 5130, 192, "sp24_skinny_m64_a32"),
          # 5 to 16 rows with eight waves (nine or more load groups of K),
          # a partial last group, and all 16 staged rows of B in use or not
          (12, 3000, 4160, "sp24_skinny_m16"), (16, 6150, 4096, "sp24_skinny_m16_a32"),
          (13, 24600, 4160, "sp24_skinny_m16_a32")]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3])
@pytest.mark.parametrize("M,N,K,kernel", SKINNY)
def test_skinny_variants_exact(dt, M, N, K, kernel):
    """Every kernel variant of the few-row range on exact-integer inputs:
    bitwise equal to the oracle."""
    K = K if dt != oracle.E4M3 else 2 * K
    ttype = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.E4M3: torch.float8_e4m3fn}[dt]
    assert sp.gemm_kernel(True, sp.SPARSE_W, ttype, torch.float32, M, N, K) == kernel
    say("skinny", kernel, dt, M, N, K)
    Y, R, _ = _sparse_w(dt, oracle.F32, M, N, K, seed=M * 7 + N, integer=True)
    assert np.array_equal(Y, R)


DENSE_FEW = [(40, 17000, 704, "dense_big_128x64"), (17, 61500, 200, "dense_big_256x64"),
             (64, 190, 704, "dense_skinny_m4"), (20, 300, 200, "dense_skinny_m2"),
             (64, 5200, 704, "dense_skinny_m4_a32"), (20, 6150, 200, "dense_skinny_m2_a32"),
             # 5 to 16 rows staged in LDS: partial last step, eight waves, 32-row tiles
             (9, 300, 200, "dense_skinny_m16"), (12, 3000, 4160, "dense_skinny_m16"),
             (16, 6150, 4096, "dense_skinny_m16_a32"), (13, 24600, 4168, "dense_skinny_m16_a32")]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3])
@pytest.mark.parametrize("M,N,K,kernel", DENSE_FEW)
def test_dense_few_rows_exact(dt, M, N, K, kernel):
    """The dense kernels of the few-row range (tile kernels on wide outputs,
    the K-splitting kernel otherwise), with a partial last K step, on
    exact-integer inputs: bitwise equal to the oracle."""
    K = K if dt != oracle.E4M3 else 2 * K
    ttype = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.E4M3: torch.float8_e4m3fn}[dt]
    assert sp.gemm_kernel(False, sp.SPARSE_W, ttype, torch.float32, M, N, K) == kernel
    say("dense few", kernel, dt, M, N, K)
    Y, R, _ = _dense(dt, oracle.F32, M, N, K, seed=M * 11 + N, integer=True)
    assert np.array_equal(Y, R)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.E4M3])
@pytest.mark.parametrize("M,N,K", [(3, 40, 96), (16, 17, 200), (100, 70, 112), (130, 129, 1040)])
def test_dense_accepts_k_the_sparse_path_rejects(dt, M, N, K):
    """The dense fallback takes any K filling whole 16-byte row chunks, so a
    partial last K step is read as zeros."""
    if dt == oracle.E4M3:
        K = (K + 15) // 16 * 16
    say("dense K tail", dt, M, N, K)
    Y, R, _ = _dense(dt, oracle.F32, M, N, K, seed=K + M, integer=True, prune_w=False)
    assert np.array_equal(Y, R)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3])
@pytest.mark.parametrize("which", ["sparse_w", "sparse_x", "dense"])
@pytest.mark.parametrize("steps", [6, 7])
@pytest.mark.parametrize("MN", [(3000, 4100), (3000, 3000), (2000, 4000), (1500, 2040), (600, 1000)])
def test_large_tile_kernels_ragged(dt, which, steps, MN):
    """The LDS-staged tile kernels (256x256, 256x128, 128x128 and 128x64,
    sparse and dense, by the tile rule on these shapes) on ragged last tiles
    in both dimensions (and, for dense, a partial last K step), with an even
    and an odd count of K steps (the sparse kernels load metadata in blocks of
    four 16-bit or two fp8 steps).  Integer inputs: sampled rows must match
    the oracle exactly."""
    M, N = MN
    K = steps * (64 if dt != oracle.E4M3 else 128)
    if which == "dense":
        K += 16                     # not a whole 64-K (128-K) step
    say("large ragged", which, dt, M, N, K)
    xb, _, wb, _ = _operands(dt, M, N, K, 123, integer=True)
    rows = np.array([0, 1, 255, 256, M // 2 + 1, M - 1])
    X, W = to_dev(xb, dt), to_dev(wb, dt)
    if which == "sparse_w":
        wv, wm = oracle.prune_compress(dt, wb)
        R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, mrows=rows)
        v, m = sp.prune_compress(W)
        Y = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out_dtype=torch.float32)
    elif which == "sparse_x":
        xv, xm = oracle.prune_compress(dt, xb)
        R = oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, mrows=rows)
        v, m = sp.prune_compress(X)
        Y = sp.sp24_gemm(sp.SPARSE_X, v, m, W, M, N, K, out_dtype=torch.float32)
    else:
        R = oracle.gemm(dt, M, N, K, x=xb, w=wb, mrows=rows)
        Y = sp.dense_gemm(X, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(decode_out(Y[torch.from_numpy(rows).cuda()]), R)


@pytest.mark.parametrize("dt,out", [(oracle.BF16, oracle.BF16), (oracle.F16, oracle.F16), (oracle.BF16, oracle.F16)])
@pytest.mark.parametrize("which", ["sparse_w", "sparse_x", "dense"])
@pytest.mark.parametrize("MN", [(4096, 3072), (3900, 3016), (3000, 4100)])
def test_staged_epilogue_16bit_exact(dt, out, which, MN):
    """16-bit outputs of the tile kernels, whose epilogue stages whole wave
    blocks in LDS and writes 16-byte pieces of output rows (along either
    operand's dimension), with direct stores for blocks cut by the edge and
    for row strides that are not a multiple of 8 (N = 4100).  Integer
    inputs keep every sum exact in fp32, so each output must be the RNE
    encoding of the oracle's value, bit for bit."""
    M, N = MN
    K = 256
    say("staged epilogue", which, dt, out, M, N, K)
    xb, _, wb, _ = _operands(dt, M, N, K, 321, integer=True)
    rows = np.array([0, 1, 15, 16, 255, 256, 257, M // 2 + 3, M - 2, M - 1])
    X, W = to_dev(xb, dt), to_dev(wb, dt)
    if which == "sparse_w":
        wv, wm = oracle.prune_compress(dt, wb)
        R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, mrows=rows)
        v, m = sp.prune_compress(W)
        Y = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out_dtype=OUT_T[out])
    elif which == "sparse_x":
        xv, xm = oracle.prune_compress(dt, xb)
        R = oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, mrows=rows)
        v, m = sp.prune_compress(X)
        Y = sp.sp24_gemm(sp.SPARSE_X, v, m, W, M, N, K, out_dtype=OUT_T[out])
    else:
        wb = oracle.prune(dt, wb)
        R = oracle.gemm(dt, M, N, K, x=xb, w=wb, mrows=rows)
        Y = sp.dense_gemm(X, to_dev(wb, dt), out_dtype=OUT_T[out])
    torch.cuda.synchronize()
    got = Y[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.encode(out, R))


# 256x256 grids with a short last round, whose remainder runs as quarter
# tiles: (M, N, K steps) with ragged last tiles in both dimensions
TAIL = [(4066, 4302, 6), (4096, 5120 - 40, 7), (1000, 68 * 256 - 7, 5)]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3])
@pytest.mark.parametrize("which", ["sparse_w", "sparse_x", "dense"])
@pytest.mark.parametrize("M,N,steps", TAIL)
def test_tail_quarter_tiles(dt, which, M, N, steps):
    """The 256x256 kernels (sparse and dense) with their last round split
    into 128x128 quarter tiles: integer inputs, rows sampled from every
    256-row band of the output (both halves of each), bitwise equal to the
    oracle, and every output written."""
    _tail_case(dt, which, M, N, steps, quarters=True)


# remainders of 65 to 128 tiles, whose halves (256x128, split along B) fill
# one round: (M, N, K steps) with ragged last tiles in both dimensions
TAIL_HALVES = [(2048 - 7, 28672 - 40, 6), (4093, 5276, 7)]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.E4M3])
@pytest.mark.parametrize("which", ["sparse_w", "sparse_x", "dense"])
@pytest.mark.parametrize("M,N,steps", TAIL_HALVES)
def test_tail_half_tiles(dt, which, M, N, steps):
    """The same with the last round split into 256x128 half tiles."""
    _tail_case(dt, which, M, N, steps, quarters=False)


def _tail_case(dt, which, M, N, steps, quarters):
    K = steps * (64 if dt != oracle.E4M3 else 128)
    RA, RB = (M, N) if which == "sparse_x" else (N, M)
    t = ((RA + 255) // 256) * ((RB + 255) // 256)
    if quarters:
        assert t > 256 and 0 < t % 256 <= 64, t
    else:
        assert t > 256 and 64 < t % 256 <= 128, t
    ttype = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.E4M3: torch.float8_e4m3fn}[dt]
    op = sp.SPARSE_X if which == "sparse_x" else sp.SPARSE_W
    name = "dense_big_256x256_tail" if which == "dense" else "sp24_big_256x256_tail"
    assert sp.gemm_kernel(which != "dense", op, ttype, torch.float32, M, N, K) == name
    say("tail quarters" if quarters else "tail halves", which, dt, M, N, K)
    xb, _, wb, _ = _operands(dt, M, N, K, 321, integer=True)
    rows = np.unique(np.clip(np.concatenate([np.arange(0, M, 256), np.arange(129, M, 256),
                                             np.arange(255, M, 256), [M - 1]]), 0, M - 1))
    X, W = to_dev(xb, dt), to_dev(wb, dt)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    if which == "sparse_w":
        wv, wm = oracle.prune_compress(dt, wb)
        R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, mrows=rows)
        v, m = sp.prune_compress(W)
        sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out=Y)
    elif which == "sparse_x":
        xv, xm = oracle.prune_compress(dt, xb)
        R = oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, mrows=rows)
        v, m = sp.prune_compress(X)
        sp.sp24_gemm(sp.SPARSE_X, v, m, W, M, N, K, out=Y)
    else:
        R = oracle.gemm(dt, M, N, K, x=xb, w=wb, mrows=rows)
        sp.dense_gemm(X, W, out=Y)
    torch.cuda.synchronize()
    assert np.array_equal(decode_out(Y[torch.from_numpy(rows).cuda()]), R)
    # every tile wrote its outputs: none is left at the NaN it started with
    assert torch.isfinite(Y).all()


def test_one_hot_rows_read_back_weights():
    """X = identity rows: Y[m, :] is column m of the decompressed W, which
    checks every metadata position and word through the sparse MMA."""
    dt, K, N = oracle.BF16, 256, 96
    wb = inputs.to_bits(inputs.normal((N, K), 1.0, 3), dt)
    v, m = sp.prune_compress(to_dev(wb, dt))
    for M0 in (0, 64):           # skinny (M = 64) and tiled (M = 128) kernels
        M = 64 if M0 == 0 else 128
        eye = torch.zeros((M, K), dtype=torch.float32)
        for i in range(M):
            eye[i, (i + M0) % K] = 1.0
        X = to_dev(inputs.to_bits(eye, dt), dt)
        Y = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out_dtype=torch.float32)
        torch.cuda.synchronize()
        wp = oracle.decode(dt, oracle.prune(dt, wb))
        cols = [(i + M0) % K for i in range(M)]
        assert np.array_equal(decode_out(Y), wp[:, cols].T)


# ------------------------------------------------------------------ full size

def _sample_rows(M):
    """One row from every 256-row band of M (a seeded place in the band, so
    that every band of tiles is checked), plus the first and the last row."""
    return band_rows(M)


@functools.lru_cache(maxsize=1)
def _full_weight(wl, s):
    """A workload's weight (bits, scales) and the oracle's compressed form of
    it, kept for the next M of the same shape."""
    dt = inputs.WORKLOADS[wl]["dtype"]
    wb, sw = inputs.weight(wl, s)
    wv, wm = oracle.prune_compress(dt, wb)
    return wb, sw, wv, wm


FULL = []
for wl in ("tiny", "decode", "prefill", "fp8"):
    w = inputs.WORKLOADS[wl]
    for s in range(len(w["shapes"])):
        for j in range(len(w["ms"])):
            FULL.append((wl, s, j))


@pytest.mark.parametrize("wl,s,j", FULL)
def test_full_size_sparse_and_dense(wl, s, j):
    w = inputs.WORKLOADS[wl]
    dt, out = w["dtype"], w["out"]
    N, K = w["shapes"][s]
    M = w["ms"][j]
    say("full", wl, (N, K), "M", M)
    wb, sw, wv, wm = _full_weight(wl, s)
    xb, sx = inputs.activation(wl, s, j)
    rows = np.arange(M) if M <= 16 else _sample_rows(M)
    R = oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw, mrows=rows)
    W = to_dev(wb, dt)
    X = to_dev(xb, dt)
    dsx = None if sx is None else torch.from_numpy(sx).cuda()
    dsw = None if sw is None else torch.from_numpy(sw).cuda()
    v, m = sp.prune_compress(W)
    Y = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, N, K, out_dtype=OUT_T[out], scale_x=dsx, scale_w=dsw)
    Wp = sp.decompress(v, m, K)
    Yd = sp.dense_gemm(X, Wp, out_dtype=OUT_T[out], scale_x=dsx, scale_w=dsw)
    torch.cuda.synchronize()
    rt = torch.from_numpy(rows).cuda()
    e_s = oracle.relative_error(decode_out(Y[rt]), R)
    e_d = oracle.relative_error(decode_out(Yd[rt]), R)
    say("  rel err sparse", e_s, "dense", e_d)
    assert e_s <= TOL[dt] and e_d <= TOL[dt]
    # every output, not only the sampled rows, is finite
    assert bool(torch.isfinite(Y.float()).all()) and bool(torch.isfinite(Yd.float()).all())


def test_full_size_online_activation():
    dt = oracle.BF16
    M, N, K = 4096, 4096, 4096
    say("full online", M, N, K)
    xb, _ = inputs.activation("online", 0, 0)
    wb, _ = inputs.weight("online", 0)
    xv, xm = oracle.prune_compress(dt, xb)
    rows = _sample_rows(M)
    R = oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, mrows=rows)
    X = to_dev(xb, dt)
    W = to_dev(wb, dt)
    v, m = sp.prune_compress(X)
    Y = sp.sp24_gemm(sp.SPARSE_X, v, m, W, M, N, K)
    Yd = sp.dense_gemm(X, W)
    torch.cuda.synchronize()
    rt = torch.from_numpy(rows).cuda()
    assert oracle.relative_error(decode_out(Y[rt]), R) <= TOL[dt]
    Rd = oracle.gemm(dt, M, N, K, x=xb, w=wb, mrows=rows)
    assert oracle.relative_error(decode_out(Yd[rt]), Rd) <= TOL[dt]


# ------------------------------------------------------------------ edge cases

def test_empty_and_zero_k():
    X = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32, 128), dtype=torch.bfloat16, device="cuda")
    v, m = sp.prune_compress(W)
    assert sp.sp24_gemm(sp.SPARSE_W, v, m, X, 0, 32, 128).shape == (0, 32)
    assert sp.dense_gemm(X, W).shape == (0, 32)
    # K = 0: the empty sum, Y = 0
    X0 = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    W0 = torch.zeros((7, 0), dtype=torch.bfloat16, device="cuda")
    v0, m0 = sp.prune_compress(W0)
    Y = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    sp.sp24_gemm(sp.SPARSE_W, v0, m0, X0, 5, 7, 0, out=Y)
    torch.cuda.synchronize()
    assert bool((Y == 0).all())


def test_ineligible_shapes_raise_align():
    X = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32, 96), dtype=torch.bfloat16, device="cuda")
    v, m = sp.prune_compress(W)
    with pytest.raises(sp.Sp24Error) as e:
        sp.sp24_gemm(sp.SPARSE_W, v, m, X, 4, 32, 96)
    assert e.value.status == 4


def test_output_guard_bands():
    dt = oracle.BF16
    for M, N, K in ((5, 40, 256), (130, 72, 256)):
        say("guard", M, N, K)
        xb, _, wb, _ = _operands(dt, M, N, K, 99)
        guard = 512
        buf = torch.full((M * N + 2 * guard,), 0x7A7A, dtype=torch.int16, device="cuda")
        Y = buf[guard:guard + M * N].view(torch.bfloat16).view(M, N)
        v, m = sp.prune_compress(to_dev(wb, dt))
        sp.sp24_gemm(sp.SPARSE_W, v, m, to_dev(xb, dt), M, N, K, out=Y)
        torch.cuda.synchronize()
        b = buf.cpu().numpy()
        assert np.all(b[:guard] == 0x7A7A) and np.all(b[-guard:] == 0x7A7A)
        Yx = buf[guard:guard + M * N].view(torch.bfloat16).view(M, N)
        sp.dense_gemm(to_dev(xb, dt), to_dev(wb, dt), out=Yx)
        torch.cuda.synchronize()
        b = buf.cpu().numpy()
        assert np.all(b[:guard] == 0x7A7A) and np.all(b[-guard:] == 0x7A7A)


def test_reruns_are_bitwise_stable():
    for M in (16, 512):
        xb, _, wb, _ = _operands(oracle.BF16, M, 1024, 2048, 7)
        X, W = to_dev(xb, oracle.BF16), to_dev(wb, oracle.BF16)
        v, m = sp.prune_compress(W)
        a = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, 1024, 2048)
        b = sp.sp24_gemm(sp.SPARSE_W, v, m, X, M, 1024, 2048)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_select_tactic_record():
    dt = oracle.BF16
    for (M, N, K, which) in ((16, 4096, 4096, sp.SPARSE_W), (512, 4096, 4096, sp.SPARSE_W),
                             (1024, 1024, 1024, sp.SPARSE_X)):
        say("tactic", M, N, K, which)
        xb, _, wb, _ = _operands(dt, M, N, K, 5)
        X, W = to_dev(xb, dt), to_dev(wb, dt)
        if which == sp.SPARSE_W:
            v, m = sp.prune_compress(W)
            rec = sp.select_tactic(which, v, m, X, sp.decompress(v, m, K), M, N, K, reps=10)
        else:
            v = torch.empty((M, K // 2), dtype=torch.bfloat16, device="cuda")
            m = torch.empty((M, K // 32), dtype=torch.int32, device="cuda")
            rec = sp.select_tactic(which, v, m, W, X, M, N, K, reps=10)
            assert rec["t_compress_us"] > 0
        say("  ", rec)
        assert rec["eligible"]
        assert (rec["selected"] == "sparse") == (rec["ratio"] > 1.0)
        assert rec["t_sparse_us"] > 0 and rec["t_dense_us"] > 0
        assert rec["kernel"].startswith("sp24_" if rec["selected"] == "sparse" else "dense_")
    # ineligible shape: dense with the alignment reason
    X = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32, 96), dtype=torch.bfloat16, device="cuda")
    v, m = sp.prune_compress(W)
    rec = sp.select_tactic(sp.SPARSE_W, v, m, X, W, 4, 32, 96, reps=3)
    assert not rec["eligible"] and rec["selected"] == "dense" and rec["reason"] == "Alignment failure"
