"""GPU parity of the row-split hybrid GEMM (one launch: the first N_s weight
rows compressed, the next N_d dense; "Production 2:4 Structured Sparsity for
LLMs", section "Dense Fallback and Hybrid Sparsity Design") against the
oracle's block products, over every tile shape the launch picks, ragged
regions, both empty-region cases, fp8 with scales, and bitwise on integer
operands."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, decode_out, meta_dev, say, to_dev

pytestmark = pytest.mark.gpu

OUT = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.F32: torch.float32}


def _operands(dt, M, NS, ND, K, seed, integer=False):
    if dt == oracle.E4M3:
        x, sx = inputs.quantize_e4m3_rows(inputs.normal((M, K), 1.0, seed))
        w, sw = inputs.quantize_e4m3_rows(inputs.normal((NS + ND, K), 0.02, seed + 1))
    else:
        gen = (lambda s, seed_: torch.randint(-2, 3, s, generator=torch.Generator().manual_seed(seed_)).float()) \
            if integer else (lambda s, seed_: inputs.normal(s, 1.0 if s[0] == M else 0.02, seed_))
        x, w = inputs.to_bits(gen((M, K), seed), dt), inputs.to_bits(gen((NS + ND, K), seed + 1), dt)
        sx = sw = None
    v, m = oracle.prune_compress(dt, w[:NS])
    return x, w[NS:], v, m, sx, sw


def _run(dt, out_dt, M, NS, ND, K, seed, sample=None, integer=False):
    x, wd, v, m, sx, sw = _operands(dt, M, NS, ND, K, seed, integer)
    name = sp.hybrid_kernel(oracle_torch(dt), OUT[out_dt], M, NS, ND, K)
    say("hybrid", dt, out_dt, M, NS, ND, K, name)
    dev = lambda a, d: None if a is None or a.size == 0 else to_dev(a, d)
    tf = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    Y = sp.hybrid_gemm(dev(v, dt), meta_dev(m) if NS else None, dev(wd, dt), dev(x, dt), NS, ND,
                       out_dtype=OUT[out_dt], scale_x=tf(sx), scale_w=tf(sw))
    torch.cuda.synchronize()
    rows = np.arange(M) if sample is None else np.unique(np.r_[0, M - 1, np.random.default_rng(seed).integers(0, M, sample)])
    R = oracle.hybrid_gemm(dt, len(rows), NS, ND, K, x=x[rows], ws_vals=v, ws_meta=m, wd=wd,
                           scale_x=None if sx is None else sx[rows], scale_w=sw)
    return decode_out(Y)[rows], R, name


def oracle_torch(dt):
    return {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.E4M3: torch.float8_e4m3fn}[dt]


# (in, out, M, N_s, N_d, K): 128x128 tiles with every edge ragged and an odd step
# count; 256x128 and 256x256 tiles (sampled rows); the 256x64 / 128x64 tiles of
# M <= 64; one region empty each way
CASES = [
    (oracle.BF16, oracle.BF16, 300, 520, 264, 448),
    (oracle.F16, oracle.F32, 40, 1024, 392, 1024),
    (oracle.BF16, oracle.BF16, 64, 12288, 1000, 256),
    (oracle.BF16, oracle.BF16, 48, 49152, 520, 128),
    (oracle.BF16, oracle.BF16, 1536, 2048, 1024, 512),
    (oracle.BF16, oracle.BF16, 1000, 2048, 768, 512),
    (oracle.BF16, oracle.BF16, 2048, 4096, 1024, 256),
    (oracle.BF16, oracle.BF16, 200, 0, 776, 320),
    (oracle.F16, oracle.F16, 130, 648, 0, 256),
]


@pytest.mark.parametrize("dt,out,M,NS,ND,K", CASES)
def test_hybrid_matches_oracle(dt, out, M, NS, ND, K):
    Y, R, name = _run(dt, out, M, NS, ND, K, M + NS + ND + K, sample=48 if M >= 1024 else None)
    assert oracle.relative_error(Y, R) <= TOL[dt], name


@pytest.mark.parametrize("M,NS,ND", [(2048, 4096, 2176), (2304 - 20, 7424, 128 - 8)])
def test_hybrid_tail_quarter_tiles(M, NS, ND):
    """A hybrid grid of 256x256 tiles just past one round (264 and 270
    tiles): the remainder runs as quarter tiles, dense ones only in the first
    case, compressed and dense in the second.  Integer operands: sampled rows
    bitwise equal to the oracle, and every output written."""
    K = 256
    name = sp.hybrid_kernel(torch.bfloat16, torch.float32, M, NS, ND, K)
    assert name == "sp24_hybrid_256x256_tail", name
    x, wd, v, m, sx, sw = _operands(oracle.BF16, M, NS, ND, K, 11 + M, integer=True)
    say("hybrid tail", M, NS, ND, K)
    Y = torch.full((M, NS + ND), float("nan"), dtype=torch.float32, device="cuda")
    sp.hybrid_gemm(to_dev(v, oracle.BF16), meta_dev(m), to_dev(wd, oracle.BF16), to_dev(x, oracle.BF16),
                   NS, ND, out=Y)
    torch.cuda.synchronize()
    assert torch.isfinite(Y).all()
    rows = np.unique(np.clip(np.concatenate([np.arange(0, M, 256), np.arange(129, M, 256), [M - 1]]), 0, M - 1))
    R = oracle.hybrid_gemm(oracle.BF16, len(rows), NS, ND, K, x=x[rows], ws_vals=v, ws_meta=m, wd=wd)
    assert np.array_equal(decode_out(Y)[rows], R)


@pytest.mark.parametrize("M,NS,ND", [(260, 256, 136), (32, 512, 200)])
def test_hybrid_fp8_with_scales(M, NS, ND):
    Y, R, name = _run(oracle.E4M3, oracle.BF16, M, NS, ND, 1024, 7 + M)
    assert oracle.relative_error(Y, R) <= TOL[oracle.E4M3], name


@pytest.mark.parametrize("M,NS,ND,K", [(96, 264, 136, 512), (2048, 4096, 1024, 256)])
def test_hybrid_integer_operands_are_exact(M, NS, ND, K):
    """Small-integer operands with fp32 output: every partial sum is exact, so
    both regions (the dense one as two 2:4 halves) match the oracle bitwise."""
    Y, R, name = _run(oracle.BF16, oracle.F32, M, NS, ND, K, 3 + M, integer=True)
    assert np.array_equal(Y, R), name


def test_hybrid_dense_region_equals_the_plain_gemms():
    """The same rows through the hybrid's regions and the plain entry points:
    the compressed block against sp24_gemm, the dense block against dense_gemm
    (within the bar: the dense block adds in another order)."""
    dt, M, NS, ND, K = oracle.BF16, 512, 1024, 512, 1024
    x, wd, v, m, _, _ = _operands(dt, M, NS, ND, K, 11)
    X, V, Mt, Wd = to_dev(x, dt), to_dev(v, dt), meta_dev(m), to_dev(wd, dt)
    Y = sp.hybrid_gemm(V, Mt, Wd, X, NS, ND)
    Ys = sp.sp24_gemm(sp.SPARSE_W, V, Mt, X, M, NS, K)
    Yd = sp.dense_gemm(X, Wd)
    torch.cuda.synchronize()
    assert oracle.relative_error(decode_out(Y[:, :NS]), decode_out(Ys)) <= TOL[dt]
    assert oracle.relative_error(decode_out(Y[:, NS:]), decode_out(Yd)) <= TOL[dt]
