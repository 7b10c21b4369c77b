"""GPU parity of the K-split hybrid GEMM (columns [0, K_s) of every weight row
2:4-compressed, columns [K_s, K) dense, one launch) against the oracle's
product over the assembled weight:

  - every tile shape the dispatcher picks, ragged edges in both output
    dimensions, every input dtype, and 16-bit / fp32 outputs;
  - exact-integer inputs, where fp32 accumulation is exact in any order: the
    fp32 output equals the oracle bit for bit;
  - the degenerate splits (all 2:4, all dense);
  - every case of the ksplit bench workload at full size, one row from every
    256-row band of M."""
import functools

import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, band_rows, decode_out, meta_dev, say, to_dev

pytestmark = pytest.mark.gpu

TT = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.E4M3: torch.float8_e4m3fn,
      oracle.I8: torch.int8}
OUT = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.F32: torch.float32}


def _ints(shape, seed, lo=-3, hi=3):
    return torch.from_numpy(np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32))


def _operands(dt, M, N, K, seed, integer):
    """(x bits, w bits, scales) for a K-split GEMM."""
    if dt == oracle.I8:
        lo, hi = (-3, 3) if integer else (-127, 127)
        x = np.random.default_rng(seed).integers(lo, hi + 1, size=(M, K)).astype(np.int8).view(np.uint8)
        w = np.random.default_rng(seed + 1).integers(lo, hi + 1, size=(N, K)).astype(np.int8).view(np.uint8)
        return x, w, None, None
    if integer:
        return inputs.to_bits(_ints((M, K), seed), dt), inputs.to_bits(_ints((N, K), seed + 1), dt), None, None
    if dt == oracle.E4M3:
        x, sx = inputs.quantize_e4m3_rows(inputs.normal((M, K), 1.0, seed))
        w, sw = inputs.quantize_e4m3_rows(inputs.normal((N, K), 0.02, seed + 1))
        return x, w, sx, sw
    return inputs.to_bits(inputs.normal((M, K), 1.0, seed), dt), \
        inputs.to_bits(inputs.normal((N, K), 0.02, seed + 1), dt), None, None


def _f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _run(dt, out, M, N, KS, K, seed, integer=False, rows=None):
    x, w, sx, sw = _operands(dt, M, N, K, seed, integer)
    ws, wd = np.ascontiguousarray(w[:, :KS]), np.ascontiguousarray(w[:, KS:])
    v, m = oracle.prune_compress(dt, ws)
    name = sp.ksplit_kernel(TT[dt], OUT[out], M, N, KS, K)
    say("ksplit", dt, out, M, N, KS, K, name)
    Y = sp.ksplit_gemm(to_dev(v, dt) if KS else None, meta_dev(m) if KS else None,
                       to_dev(wd, dt) if KS < K else None, to_dev(x, dt), N, KS, out_dtype=OUT[out],
                       scale_x=_f32(sx), scale_w=_f32(sw))
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    R = oracle.ksplit_gemm(dt, M, N, KS, K, x=x, ws_vals=v, ws_meta=m, wd=wd, scale_x=sx, scale_w=sw,
                           mrows=rows)
    Yh = decode_out(Y)
    assert np.isfinite(Yh).all()
    return Yh[rows], R, name


# (M, N, K_s, K): 128x64 tiles with ragged edges; 256x64 (M <= 64, wide N);
# 128x128; 256x128; 256x256 with ragged N; the 256x256 grid with a quarter-tile
# tail (544 tiles = 2 * 256 + 32) and with a half-tile tail (336 = 256 + 80,
# ragged in both dimensions); a 2:4 range shorter than the dense one
CASES = [(40, 200, 256, 512), (64, 49408, 256, 512), (1600, 2048, 256, 1024), (2048, 3072, 768, 1024),
         (2816, 4500, 512, 1024), (8192, 4352, 256, 512), (4093, 5276, 256, 512), (300, 520, 256, 1280)]
KERNELS = ["sp24_ksplit_128x64", "sp24_ksplit_256x64", "sp24_ksplit_128x128", "sp24_ksplit_256x128",
           "sp24_ksplit_256x256", "sp24_ksplit_256x256_tail", "sp24_ksplit_256x256_tail", "sp24_ksplit_128x64"]


def test_cases_cover_every_tile_shape():
    for (M, N, KS, K), name in zip(CASES, KERNELS):
        assert sp.ksplit_kernel(torch.bfloat16, torch.bfloat16, M, N, KS, K) == name


@pytest.mark.parametrize("dt,out", [(oracle.BF16, oracle.BF16), (oracle.F16, oracle.F32), (oracle.E4M3, oracle.BF16),
                                    (oracle.I8, oracle.BF16)])
@pytest.mark.parametrize("M,N,KS,K", CASES)
def test_ksplit_matches_oracle(dt, out, M, N, KS, K):
    if dt in (oracle.E4M3, oracle.I8) and K % 128:
        K += 128 - K % 128
    rows = None if M <= 1024 else band_rows(M, seed=N)
    Y, R, _ = _run(dt, out, M, N, KS, K, seed=M + N + KS, rows=rows)
    assert oracle.relative_error(Y, R) <= TOL[dt]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16, oracle.E4M3, oracle.I8])
@pytest.mark.parametrize("M,N,KS,K", [(48, 300, 256, 768), (520, 264, 512, 1024), (2048, 4352, 256, 512)])
def test_ksplit_exact_integers(dt, M, N, KS, K):
    """|sums| < 2^24: the fp32 output equals the oracle exactly."""
    rows = None if M <= 520 else band_rows(M, seed=KS)
    Y, R, _ = _run(dt, oracle.F32, M, N, KS, K, seed=7 + M, integer=True, rows=rows)
    assert np.array_equal(Y, R)


@pytest.mark.parametrize("KS", [0, 512])
def test_ksplit_degenerate_ranges(KS):
    """All dense (K_s = 0) and all 2:4 (K_s = K), bit-exact on integers."""
    Y, R, _ = _run(oracle.BF16, oracle.F32, 300, 520, KS, 512, seed=3 + KS, integer=True)
    assert np.array_equal(Y, R)


@functools.lru_cache(maxsize=1)
def _ksplit_weight(s):
    N, K = inputs.WORKLOADS["ksplit"]["shapes"][s]
    KS, KD = inputs.ksplit_split(K)
    wb, _ = inputs.weight("ksplit", s)
    ws, wd = np.ascontiguousarray(wb[:, :KS]), np.ascontiguousarray(wb[:, KS:])
    wv, wm = oracle.prune_compress(oracle.BF16, ws)
    return wb, ws, wd, wv, wm, KS


@pytest.mark.parametrize("s,j", [(s, j) for s in range(4) for j in range(2)])
def test_ksplit_full_size(s, j):
    w = inputs.WORKLOADS["ksplit"]
    N, K = w["shapes"][s]
    M = w["ms"][j]
    wb, ws, wd, wv, wm, KS = _ksplit_weight(s)
    name = sp.ksplit_kernel(torch.bfloat16, torch.bfloat16, M, N, KS, K)
    say("full ksplit", (N, K), "K_s", KS, "M", M, name)
    xb, _ = inputs.activation("ksplit", s, j)
    Ws = to_dev(ws, oracle.BF16)
    v, m = sp.prune_compress(Ws)
    Y = sp.ksplit_gemm(v, m, to_dev(wd, oracle.BF16), to_dev(xb, oracle.BF16), N, KS)
    torch.cuda.synchronize()
    rows = band_rows(M, seed=10 * s + j)
    R = oracle.ksplit_gemm(oracle.BF16, M, N, KS, K, x=xb, ws_vals=wv, ws_meta=wm, wd=wd, mrows=rows)
    err = oracle.relative_error(decode_out(Y[torch.from_numpy(rows).cuda()]), R)
    say("  rel err", err)
    assert err <= TOL[oracle.BF16]
    assert bool(torch.isfinite(Y.float()).all())
