"""Pins of the oracle's fused online int8 path (per-row symmetric int8
quantization ahead of the 2:4 prune; the 2:4-versus-quantization paper,
section 2 "Quantization", and 4.2 "Speed" for 2:4 with INT8).  Each pin is
something the definition fixes independently of how the oracle computes it:

  - the encoder on hand-picked quotients: ties to even, saturation at
    +-127, NaN to 0;
  - rows of integer multiples of a power of two, whose scale is exactly that
    power and whose codes are the integers themselves;
  - the row maximum lands on +-127, every code is within half a step of its
    element, codes are odd in x and monotone along a sorted row;
  - a NaN does not move the scale; an all-zero row has unit scale;
  - the quotient is formed in fp32 (elements whose fp32 and exact quotients
    round apart follow fp32);
  - the fused form keeps, in every group, the two codes of largest
    magnitude;
  - an independent implementation of the same reading (torch in fp32)
    agrees on every code and scale."""
import numpy as np
import pytest

import oracle
from semi_structured_sparse_sp24_amd import inputs


def _i8(q):
    return np.asarray(q, dtype=np.uint8).view(np.int8)


def test_encode_i8_hand_picked():
    cases = [(0.0, 0), (0.4999, 0), (0.5, 0), (0.5001, 1), (1.5, 2), (2.5, 2), (3.5, 4), (-0.5, 0),
             (-1.5, -2), (-2.5, -2), (126.5, 126), (126.51, 127), (127.0, 127), (127.49, 127), (127.5, 127),
             (130.0, 127), (1e30, 127), (-1e30, -127), (-127.6, -127), (float("inf"), 127),
             (float("-inf"), -127), (float("nan"), 0)]
    for t, want in cases:
        assert oracle.encode_i8(t) == want, (t, oracle.encode_i8(t), want)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quantize_i8_exact_multiples(dt):
    """x = k * 2^e with integers |k| <= 127 and one |k| = 127 per row: the scale
    is exactly 2^e and the codes are k."""
    rng = np.random.default_rng(5)
    k = rng.integers(-127, 128, size=(16, 96))
    k[:, 7] = np.where(rng.integers(0, 2, 16) == 1, 127, -127)
    for e in (-10, -3, 0, 2):
        x = k.astype(np.float64) * 2.0 ** e
        bits = oracle.encode(dt, x)
        assert np.array_equal(oracle.decode(dt, bits), x)      # exact in the 16-bit format
        q, s = oracle.quantize_i8_rows(dt, bits)
        assert np.all(s == np.float32(2.0 ** e))
        assert np.array_equal(_i8(q), k.astype(np.int8))


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quantize_i8_maximum_bound_symmetry_monotone(dt):
    x = inputs.normal((40, 256), 1.0, 21)
    x[5] *= 1e-3
    x[6] *= 300.0
    bits = inputs.to_bits(x, dt)
    xd = oracle.decode(dt, bits)
    q, s = oracle.quantize_i8_rows(dt, bits)
    qi = _i8(q).astype(np.int64)
    rows = np.arange(40)
    arg = np.abs(xd).argmax(axis=1)
    # the largest magnitude of each row codes to +-127, with its sign
    assert np.array_equal(qi[rows, arg], 127 * np.sign(xd[rows, arg]).astype(np.int64))
    assert np.all(np.abs(qi) <= 127)
    # at most half a step of s from the element (and a little fp32 slack)
    assert np.all(np.abs(qi * s[:, None].astype(np.float64) - xd) <= 0.5 * s[:, None] * (1 + 1e-5))
    # odd in x: negating the row negates every code, and leaves the scale
    qn, sn = oracle.quantize_i8_rows(dt, oracle.encode(dt, -xd))
    assert np.array_equal(sn, s) and np.array_equal(_i8(qn).astype(np.int64), -qi)
    # monotone: along a sorted row the codes never decrease
    srt = np.sort(xd, axis=1)
    qs, _ = oracle.quantize_i8_rows(dt, oracle.encode(dt, srt))
    assert np.all(np.diff(_i8(qs).astype(np.int64), axis=1) >= 0)


def test_quantize_i8_zero_row_nan_and_inf():
    zero = np.zeros((1, 32), dtype=np.uint16)
    q, s = oracle.quantize_i8_rows(oracle.BF16, zero)
    assert s[0] == 1.0 and not q.any()
    x = oracle.decode(oracle.BF16, inputs.to_bits(inputs.normal((1, 32), 1.0, 4), oracle.BF16))[0]
    clean = oracle.encode(oracle.BF16, x)
    qc, _ = oracle.quantize_i8_rows(oracle.BF16, clean[None, :])
    big = int(np.abs(x).argmax())
    # a NaN first, last, just after the maximum, or in place of it: the scale is the
    # maximum of the other elements, and the NaN codes to 0
    for pos in sorted({0, 31, min(big + 1, 31), big}):
        row = clean.copy()
        row[pos] = 0x7fc0
        q, s = oracle.quantize_i8_rows(oracle.BF16, row[None, :])
        rest = np.delete(np.abs(x), pos).max()
        assert s[0] == np.float32(rest) / np.float32(127), pos
        assert _i8(q[0])[pos] == 0
        if pos != big:                                      # the maximum stays: the other codes stay
            others = np.arange(32) != pos
            assert np.array_equal(q[0][others], qc[0][others])
    inf = np.zeros((1, 32), dtype=np.uint16)
    inf[0, :] = oracle.encode(oracle.BF16, np.linspace(-3, 3, 32))
    inf[0, 9] = 0x7f80                                      # +inf: the scale is inf
    q, s = oracle.quantize_i8_rows(oracle.BF16, inf)
    assert np.isinf(s[0]) and not q.any()                    # finite / inf = 0; inf / inf = NaN -> 0


def test_quantize_i8_decides_codes_in_fp32():
    """Search bf16 rows for elements whose fp32 quotient x / s and whose exact
    quotient round to different integers; the oracle follows fp32."""
    all_bf16 = np.arange(0, 0x7f80, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode(oracle.BF16, all_bf16)
    found = 0
    for amax_bits in range(0x3f81, 0x3fff, 3):
        amax = oracle.decode(oracle.BF16, np.array([amax_bits], dtype=np.uint16))[0]
        s = np.float32(amax) / np.float32(127)
        cand = all_bf16[(vals > 0) & (vals < amax)]
        cv = oracle.decode(oracle.BF16, cand)
        q32 = (cv.astype(np.float32) / s).astype(np.float32)
        exact = cv / np.float64(s)
        r32, r64 = np.rint(q32.astype(np.float64)), np.rint(exact)
        diff = np.flatnonzero(r32 != r64)
        if len(diff) == 0:
            continue
        row = np.zeros((1, 32), dtype=np.uint16)
        row[0, 0] = amax_bits
        row[0, 1:1 + min(31, len(diff))] = cand[diff[:31]]
        q, sc = oracle.quantize_i8_rows(oracle.BF16, row)
        assert sc[0] == s
        n = 1 + min(31, len(diff))
        assert np.array_equal(_i8(q[0, 1:n]).astype(np.int64), r32[diff[:31]].astype(np.int64))
        found += 1
        if found >= 3:
            break
    assert found >= 1, "no element found whose fp32 and fp64 quotients round apart"


def test_quantize_i8_prune_compress_keeps_the_largest_codes():
    x = inputs.normal((8, 128), 1.0, 6)
    bits = inputs.to_bits(x, oracle.BF16)
    v, m, s = oracle.quantize_i8_prune_compress(oracle.BF16, bits)
    q, s2 = oracle.quantize_i8_rows(oracle.BF16, bits)
    assert np.array_equal(s, s2)
    dense = oracle.decompress(oracle.I8, v, m, 128)
    qa = np.abs(_i8(q).astype(np.int64)).reshape(8, 32, 4)
    da = np.abs(_i8(dense).astype(np.int64)).reshape(8, 32, 4)
    # in every group the two kept magnitudes are the two largest of the codes
    assert np.array_equal(np.sort(da, axis=2)[:, :, 2:], np.sort(qa, axis=2)[:, :, 2:])
    # and the kept codes are codes of the row at their positions
    assert np.all((_i8(dense) == 0) | (_i8(dense) == _i8(q)))


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quantize_i8_matches_torch_fp32(dt):
    """An independent implementation of the same reading: torch's fp32 maximum,
    division by 127 and by the scale (IEEE, correctly rounded), round half to
    even and clamp, on the decoded rows (outliers included, no NaN)."""
    import torch
    x = inputs.outliers(inputs.normal((64, 512), 1.0, 31), 0.01, 20.0, 32)
    bits = inputs.to_bits(x, dt)
    xd = torch.from_numpy(oracle.decode(dt, bits)).to(torch.float32)
    amax = xd.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
    qt = torch.round(xd / s[:, None]).clamp(-127, 127).to(torch.int8)
    q, sc = oracle.quantize_i8_rows(dt, bits)
    assert np.array_equal(sc, s.numpy())
    assert np.array_equal(_i8(q), qt.numpy())
