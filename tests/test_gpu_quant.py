"""GPU parity of the fused online fp8 path (per-row e4m3 quantization with the
2:4 prune and compress, and the plain quantization of the dense side) against
the oracle: codes, metadata and scales byte for byte; then the fp8 sparse
GEMM on the fused output against the oracle's product."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import TOL, decode_out, say, to_dev

pytestmark = pytest.mark.gpu

# rows held by one wave (K <= 4096, 1, 2 or 4 chunks a lane), by two waves
# (the last workgroup of an odd row count half idle), by four waves, and rows
# long enough to be taken in two rounds
SHAPES = [(1, 32), (3, 96), (5, 1024), (67, 1056), (130, 4096), (9, 4128), (3, 12288), (2, 20480),
          (2, 36864)]


def _bits(dt, rows, K, seed, outliers=False):
    x = inputs.normal((rows, K), 1.0, seed)
    if outliers:
        x = inputs.outliers(x, 0.01, 20.0, seed + 1)
    return inputs.to_bits(x, dt)


def _host(t):
    return t.view(torch.uint8).cpu().numpy() if t.dtype == torch.float8_e4m3fn else t.cpu().numpy()


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("rows,K", SHAPES)
def test_fused_matches_oracle_bytewise(dt, rows, K):
    say("quant fused", dt, rows, K)
    bits = _bits(dt, rows, K, rows * 13 + K, outliers=True)
    v, m, s = oracle.quantize_prune_compress(dt, bits)
    gv, gm, gs = sp.quantize_prune_compress(to_dev(bits, dt))
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s)
    assert np.array_equal(_host(gv), v)
    assert np.array_equal(_host(gm).view(np.uint32), m)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("rows,K", SHAPES)
def test_plain_matches_oracle_bytewise(dt, rows, K):
    say("quant plain", dt, rows, K)
    bits = _bits(dt, rows, K, rows * 17 + K)
    q, s = oracle.quantize_e4m3_rows(dt, bits)
    gq, gs = sp.quantize_e4m3(to_dev(bits, dt))
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s)
    assert np.array_equal(_host(gq), q)


# more rows than the workgroups resident at once (one row per workgroup), so
# the rows are taken in several waves of workgroups; the last shape takes two
# rounds per row
LOOP_SHAPES = [(5000, 64), (1600, 4128), (1100, 8224), (600, 16416), (520, 32800)]


@pytest.mark.parametrize("rows,K", LOOP_SHAPES)
def test_rows_walked_by_a_resident_grid(rows, K):
    say("quant loop", rows, K)
    bits = _bits(oracle.BF16, rows, K, rows + K, outliers=True)
    dev = to_dev(bits, oracle.BF16)
    v, m, s = oracle.quantize_prune_compress(oracle.BF16, bits)
    gv, gm, gs = sp.quantize_prune_compress(dev)
    q, s2 = oracle.quantize_e4m3_rows(oracle.BF16, bits)
    gq, gs2 = sp.quantize_e4m3(dev)
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s) and np.array_equal(_host(gs2), s2)
    assert np.array_equal(_host(gv), v)
    assert np.array_equal(_host(gm).view(np.uint32), m)
    assert np.array_equal(_host(gq), q)


def test_special_rows():
    """All-zero row (scale 1), a row holding one huge outlier, negative zeros,
    subnormal-range quotients, and elements whose fp32 quotient rounds to a
    different code than the exact one."""
    K = 64
    bits = np.zeros((6, K), dtype=np.uint16)
    bits[1, 7] = 0x4f80                                   # 2^32: everything else rounds to 0
    bits[1, 8] = 0x3f80
    bits[2, :] = 0x8000                                   # -0.0
    bits[3] = inputs.to_bits(inputs.normal((1, K), 1e-3, 4), oracle.BF16)[0]
    bits[3, 0] = 0x4400                                   # 512: the rest lands below the normals
    # a row found by searching the fp32 / exact quotient disagreement (see the oracle's pins)
    all_bf16 = np.arange(1, 0x7f80, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode(oracle.BF16, all_bf16)
    amax_bits = 0x3fc1
    amax = oracle.decode(oracle.BF16, np.array([amax_bits], dtype=np.uint16))[0]
    sc = np.float32(amax) / np.float32(448)
    cand = all_bf16[vals < amax]
    cv = oracle.decode(oracle.BF16, cand)
    q32 = oracle.encode_e4m3((cv.astype(np.float32) / sc).astype(np.float64))
    q64 = oracle.encode_e4m3(cv / np.float64(sc))
    diff = cand[q32 != q64]
    bits[4, 0] = amax_bits
    bits[4, 1:1 + min(K - 1, len(diff))] = diff[:K - 1]
    bits[5] = _bits(oracle.BF16, 1, K, 77)[0]
    say("quant special", len(diff))
    for fused in (True, False):
        dev = to_dev(bits, oracle.BF16)
        if fused:
            v, m, s = oracle.quantize_prune_compress(oracle.BF16, bits)
            gv, gm, gs = sp.quantize_prune_compress(dev)
            torch.cuda.synchronize()
            assert np.array_equal(_host(gv), v) and np.array_equal(_host(gm).view(np.uint32), m)
        else:
            q, s = oracle.quantize_e4m3_rows(oracle.BF16, bits)
            gq, gs = sp.quantize_e4m3(dev)
            torch.cuda.synchronize()
            assert np.array_equal(_host(gq), q)
        assert np.array_equal(_host(gs), s)


def _bits_neighbours(dt, bits):
    """The 16-bit patterns one unit below and above each pattern (same sign)."""
    b = bits.astype(np.int64)
    return np.concatenate([b - 1, b, b + 1]).astype(np.uint16)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quotients_on_and_around_e4m3_midpoints(dt):
    """Rows whose scale is a power of two (max |x| = 448 * 2^k), so x / s is
    exact and every rounding midpoint of e4m3 -- and the 16-bit values right
    next to it -- is hit: ties to even, and the elements the fast conversion
    must hand to the exact division."""
    pos = oracle.decode(oracle.E4M3, np.arange(0, 0x7f, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    rows = []
    for k in (-3, 0, 5):
        xs = mids * 2.0 ** k
        bits = _bits_neighbours(dt, oracle.encode(dt, xs))
        vals = oracle.decode(dt, bits)
        bits = bits[(np.abs(vals) < 448 * 2.0 ** k) & (vals > 0)]
        row = np.concatenate([oracle.encode(dt, np.array([448 * 2.0 ** k])), bits, bits | 0x8000])
        K = (len(row) + 31) // 32 * 32
        rows.append(np.pad(row, (0, K - len(row))))
    K = max(len(r) for r in rows)
    bits = np.stack([np.pad(r, (0, K - len(r))) for r in rows]).astype(np.uint16)
    say("quant midpoints", dt, bits.shape)
    q, s = oracle.quantize_e4m3_rows(dt, bits)
    assert np.array_equal(s, np.float32([2.0 ** -3, 1.0, 2.0 ** 5]))
    gq, gs = sp.quantize_e4m3(to_dev(bits, dt))
    v, m, _ = oracle.quantize_prune_compress(dt, bits)
    gv, gm, _ = sp.quantize_prune_compress(to_dev(bits, dt))
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s)
    assert np.array_equal(_host(gq), q)
    assert np.array_equal(_host(gv), v) and np.array_equal(_host(gm).view(np.uint32), m)


@pytest.mark.parametrize("K", [64, 8192])
def test_rows_with_infinities_and_nans(K):
    """A NaN does not count toward the row maximum and codes to 0x7f; an
    infinite maximum gives an infinite scale (finite elements code to zero,
    the infinity to NaN).  At K = 8192 two rows share a workgroup, one with a
    NaN and one without."""
    bits = inputs.to_bits(inputs.normal((5, K), 1.0, 21), oracle.BF16)
    bits[0, 5] = 0x7fc1                                   # NaN
    bits[2, 9] = 0xffc0                                   # NaN with the sign bit
    bits[3, 3] = 0x7f80                                   # +inf
    bits[4, 0] = 0xff80                                   # -inf
    say("quant inf/nan", K)
    q, s = oracle.quantize_e4m3_rows(oracle.BF16, bits)
    gq, gs = sp.quantize_e4m3(to_dev(bits, oracle.BF16))
    v, m, _ = oracle.quantize_prune_compress(oracle.BF16, bits)
    gv, gm, _ = sp.quantize_prune_compress(to_dev(bits, oracle.BF16))
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s)
    assert np.array_equal(_host(gq), q)
    assert np.array_equal(_host(gv), v) and np.array_equal(_host(gm).view(np.uint32), m)


def test_fused_output_feeds_the_fp8_sparse_gemm():
    """X (bf16, outliers) -> fused quantize+prune+compress -> sp24_gemm(SPARSE_X,
    e4m3) with W e4m3 and per-channel scales, against the oracle's product on
    the same bytes."""
    M, N, K = 300, 520, 1024
    say("quant gemm", M, N, K)
    xb = _bits(oracle.BF16, M, K, 5, outliers=True)
    wq, sw = inputs.quantize_e4m3_rows(inputs.normal((N, K), 0.02, 6))
    xv, xm, sx = oracle.quantize_prune_compress(oracle.BF16, xb)
    R = oracle.gemm(oracle.E4M3, M, N, K, x_vals=xv, x_meta=xm, w=wq, scale_x=sx, scale_w=sw)
    gv, gm, gs = sp.quantize_prune_compress(to_dev(xb, oracle.BF16))
    Y = sp.sp24_gemm(sp.SPARSE_X, gv, gm, to_dev(wq, oracle.E4M3), M, N, K, out_dtype=torch.bfloat16,
                     scale_x=gs, scale_w=torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    assert oracle.relative_error(decode_out(Y), R) <= TOL[oracle.E4M3]


def test_near_tie_words_with_negative_zero_and_tiny_elements():
    """Rows of scale 1 (max |x| = 448) whose words hold an exact e4m3 midpoint,
    so they take the exact quotient, together with -0 (its code keeps the sign)
    and elements below 2^-100 (which take the division)."""
    mid = 1.0625                       # halfway between the e4m3 values 1.0 and 1.125
    words = [[mid, -0.0, 2.0, 3.0], [mid, 2.0 ** -110, -2.0 ** -105, 5.0], [-mid, 0.0, -0.0, 2.0 ** -120],
             [mid * 4, 7.0, -2.0 ** -101, 1.0]]
    row = np.array([448.0] + [v for w in words for v in w] + [0.0] * 15)[:32]
    bits = np.stack([oracle.encode(dt_, row) for dt_ in (oracle.BF16,)])
    say("quant near-tie words", bits.shape)
    q, s = oracle.quantize_e4m3_rows(oracle.BF16, bits)
    assert s[0] == 1.0
    v, m, _ = oracle.quantize_prune_compress(oracle.BF16, bits)
    dev = to_dev(bits, oracle.BF16)
    gq, gs = sp.quantize_e4m3(dev)
    gv, gm, _ = sp.quantize_prune_compress(dev)
    torch.cuda.synchronize()
    assert np.array_equal(_host(gs), s)
    assert np.array_equal(_host(gq), q)
    assert np.array_equal(_host(gv), v) and np.array_equal(_host(gm).view(np.uint32), m)
