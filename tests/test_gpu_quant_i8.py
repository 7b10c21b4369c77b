"""GPU parity of the fused online int8 path (per-row symmetric int8
quantization with the 2:4 prune and compress, and the plain quantization of
the dense side) against the oracle: codes, metadata and scales byte for byte;
then the int8 sparse GEMM on the fused output against the oracle's product."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, decode_out, say, to_dev

pytestmark = pytest.mark.gpu

# one chunk a lane (K <= 4096), two, four, eight, and rows taken in two rounds
SHAPES = [(1, 32), (3, 96), (5, 1024), (67, 1056), (130, 4096), (9, 4128), (3, 12288), (2, 20480),
          (2, 36864)]


def _bits(dt, rows, K, seed, outliers=False):
    x = inputs.normal((rows, K), 1.0, seed)
    if outliers:
        x = inputs.outliers(x, 0.01, 20.0, seed + 1)
    return inputs.to_bits(x, dt)


def _host(t):
    return t.view(torch.uint8).cpu().numpy() if t.dtype == torch.int8 else t.cpu().numpy()


def _both(dt, bits):
    """(oracle, GPU) of the fused and the plain quantizer on the same rows, compared byte for byte."""
    v, m, s = oracle.quantize_i8_prune_compress(dt, bits)
    q, s2 = oracle.quantize_i8_rows(dt, bits)
    dev = to_dev(bits, dt)
    gv, gm, gs = sp.quantize_i8_prune_compress(dev)
    gq, gs2 = sp.quantize_i8(dev)
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s) and np.array_equal(_host(gs2), s2)
    assert np.array_equal(_host(gq), q)
    assert np.array_equal(_host(gv), v)
    assert np.array_equal(_host(gm).view(np.uint32), m)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("rows,K", SHAPES)
def test_matches_oracle_bytewise(dt, rows, K):
    say("quant i8", dt, rows, K)
    _both(dt, _bits(dt, rows, K, rows * 19 + K, outliers=True))


# more rows than the workgroups resident at once, so the rows are taken in
# several waves of workgroups; the last shape takes two rounds per row
LOOP_SHAPES = [(5000, 64), (1600, 4128), (520, 32800)]


@pytest.mark.parametrize("rows,K", LOOP_SHAPES)
def test_many_rows(rows, K):
    say("quant i8 rows", rows, K)
    _both(oracle.BF16, _bits(oracle.BF16, rows, K, rows + 3 * K, outliers=True))


def test_special_rows():
    """All-zero row (scale 1), a row holding one huge outlier, negative zeros,
    a row whose scale lies below the fp32 normals, and elements whose fp32
    quotient rounds to a different integer than the exact one."""
    K = 64
    bits = np.zeros((7, K), dtype=np.uint16)
    bits[1, 7] = 0x4f80                                   # 2^32: everything else rounds to 0
    bits[1, 8] = 0x3f80
    bits[2, :] = 0x8000                                   # -0.0
    bits[3] = inputs.to_bits(inputs.normal((1, K), 1e-3, 4), oracle.BF16)[0]
    bits[3, 0] = 0x4400                                   # 512 beside values near 1e-3
    bits[4, :8] = [0x0080, 0x0040, 0x8020, 0x0001, 0x80ff, 0x0010, 0x0000, 0x0003]   # max 2^-126: s subnormal
    # a row found by searching the fp32 / exact quotient disagreement (see the oracle's pins)
    all_bf16 = np.arange(1, 0x7f80, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode(oracle.BF16, all_bf16)
    diff = np.zeros(0, dtype=np.uint16)
    amax_bits = 0x3f81
    while len(diff) == 0:
        amax_bits += 1
        amax = oracle.decode(oracle.BF16, np.array([amax_bits], dtype=np.uint16))[0]
        sc = np.float32(amax) / np.float32(127)
        cand = all_bf16[vals < amax]
        cv = oracle.decode(oracle.BF16, cand)
        q32 = np.rint((cv.astype(np.float32) / sc).astype(np.float64))
        q64 = np.rint(cv / np.float64(sc))
        diff = cand[q32 != q64]
    bits[5, 0] = amax_bits
    bits[5, 1:1 + min(K - 1, len(diff))] = diff[:K - 1]
    bits[6] = _bits(oracle.BF16, 1, K, 77)[0]
    say("quant i8 special", len(diff))
    _both(oracle.BF16, bits)


def _bits_neighbours(bits):
    """The 16-bit patterns one unit below and above each pattern (same sign)."""
    b = bits.astype(np.int64)
    return np.concatenate([b - 1, b, b + 1]).astype(np.uint16)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quotients_on_and_around_half_integers(dt):
    """Rows whose scale is a power of two (max |x| = 127 * 2^k), so x / s is
    exact and every half-integer 0.5 .. 126.5 -- and the 16-bit values right
    next to it -- is hit: ties to even, and the elements the fast rounding must
    hand to the exact division."""
    halves = np.arange(0, 127) + 0.5
    rows = []
    for k in (-3, 0, 5):
        bits = _bits_neighbours(oracle.encode(dt, halves * 2.0 ** k))
        vals = oracle.decode(dt, bits)
        bits = bits[(np.abs(vals) < 127 * 2.0 ** k) & (vals > 0)]
        row = np.concatenate([oracle.encode(dt, np.array([127 * 2.0 ** k])), bits, bits | 0x8000])
        rows.append(row)
    K = (max(len(r) for r in rows) + 31) // 32 * 32
    bits = np.stack([np.pad(r, (0, K - len(r))) for r in rows]).astype(np.uint16)
    say("quant i8 halves", dt, bits.shape)
    q, s = oracle.quantize_i8_rows(dt, bits)
    assert np.array_equal(s, np.float32([2.0 ** -3, 1.0, 2.0 ** 5]))
    _both(dt, bits)


@pytest.mark.parametrize("K", [64, 8192])
def test_rows_with_infinities_and_nans(K):
    """A NaN does not count toward the row maximum and codes to 0; an infinite
    maximum gives an infinite scale (every code 0)."""
    bits = inputs.to_bits(inputs.normal((5, K), 1.0, 23), oracle.BF16)
    bits[0, 5] = 0x7fc1                                   # NaN
    bits[2, 9] = 0xffc0                                   # NaN with the sign bit
    bits[3, 3] = 0x7f80                                   # +inf
    bits[4, 0] = 0xff80                                   # -inf
    say("quant i8 inf/nan", K)
    _both(oracle.BF16, bits)


def test_fused_output_feeds_the_int8_sparse_gemm():
    """X (bf16, outliers) -> fused int8 quantize+prune+compress -> sp24_gemm(SPARSE_X,
    int8) with W int8 and per-channel scales, against the oracle's product on
    the same bytes."""
    M, N, K = 300, 520, 1024
    say("quant i8 gemm", M, N, K)
    xb = _bits(oracle.BF16, M, K, 8, outliers=True)
    wq, sw = inputs.quantize_i8_rows(inputs.normal((N, K), 0.02, 9))
    xv, xm, sx = oracle.quantize_i8_prune_compress(oracle.BF16, xb)
    R = oracle.gemm(oracle.I8, M, N, K, x_vals=xv, x_meta=xm, w=wq, scale_x=sx, scale_w=sw)
    gv, gm, gs = sp.quantize_i8_prune_compress(to_dev(xb, oracle.BF16))
    Y = sp.sp24_gemm(sp.SPARSE_X, gv, gm, to_dev(wq, oracle.I8), M, N, K, out_dtype=torch.bfloat16,
                     scale_x=gs, scale_w=torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    assert oracle.relative_error(decode_out(Y), R) <= TOL[oracle.I8]


def test_near_tie_words_with_negative_zero_and_tiny_elements():
    """Rows of scale 1 (max |x| = 127) whose words hold an exact half-integer,
    so they take the exact quotient, together with -0 and elements below
    2^-100 (which take the division)."""
    words = [[2.5, -0.0, 2.0, 3.0], [-3.5, 2.0 ** -110, -2.0 ** -105, 5.0], [0.5, 0.0, -0.0, 2.0 ** -120],
             [126.5, 7.0, -2.0 ** -101, 1.0]]
    row = np.array([127.0] + [v for w in words for v in w] + [0.0] * 15)[:32]
    bits = oracle.encode(oracle.BF16, row)[None, :]
    say("quant i8 near-tie words", bits.shape)
    q, s = oracle.quantize_i8_rows(oracle.BF16, bits)
    assert s[0] == 1.0
    _both(oracle.BF16, bits)
