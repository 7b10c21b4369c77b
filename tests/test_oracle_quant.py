"""Pins of the oracle's fused online fp8 path (per-row e4m3 quantization ahead
of the 2:4 prune; the 2:4-versus-quantization paper, section 2
"Quantization" and sections 3.5 / 4.2): the e4m3 encoder against torch's
cast and against a brute-force nearest-value search, its saturation, and
the row quantizer against closed forms (exact round trips, the row maximum
landing on 448, the rounding bound)."""
import numpy as np
import pytest
import torch

import oracle
from semi_structured_sparse_sp24_amd import inputs

# every finite positive e4m3 value, in code order (codes 0x00 .. 0x7e)
POS_CODES = np.arange(0, 0x7f, dtype=np.uint8)
POS_VALUES = oracle.decode(oracle.E4M3, POS_CODES)


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_e4m3_matches_torch_below_saturation():
    mids = (POS_VALUES[:-1] + POS_VALUES[1:]) / 2            # exact halfway cases (ties to even)
    f32 = mids.astype(np.float32)
    around = np.concatenate([np.nextafter(f32, np.float32(0)), f32, np.nextafter(f32, np.float32(1e9))])
    rnd = np.random.default_rng(7).uniform(-447.9, 447.9, 200_000).astype(np.float32)
    xs = np.concatenate([POS_VALUES.astype(np.float32), -POS_VALUES.astype(np.float32), around, -around, rnd])
    assert np.array_equal(oracle.encode_e4m3(xs.astype(np.float64)), _torch_e4m3(xs))


def test_encode_e4m3_is_nearest_brute_force():
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.uniform(0, 447.9, 3000), rng.uniform(0, 2.0 ** -5, 3000),
                         (POS_VALUES[:-1] + POS_VALUES[1:]) / 2])
    codes = oracle.encode_e4m3(xs)
    for x, c in zip(xs, codes):
        d = np.abs(POS_VALUES - x)
        best = np.flatnonzero(d == d.min())
        if len(best) == 1:
            assert c == best[0], (x, c, best)
        else:                                                # a tie: the even code wins
            assert c in best and c % 2 == 0, (x, c, best)


def test_encode_e4m3_saturates_and_keeps_nan():
    assert oracle.encode_e4m3(np.array([448.0, 463.9, 464.0, 470.0, 479.9, 1e30])).tolist() == [0x7e] * 6
    assert oracle.encode_e4m3(np.array([-448.0, -1e30])).tolist() == [0xfe] * 2
    assert oracle.encode_e4m3(np.array([np.nan])).tolist() == [0x7f]
    assert oracle.encode_e4m3(np.array([0.0, -0.0])).tolist() == [0x00, 0x80]


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quantize_exact_round_trip(dt):
    """Rows of e4m3 values times 2^k whose largest magnitude is 448 * 2^k:
    the scale is exactly 2^k and the codes come back unchanged."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7f, size=(12, 64), dtype=np.uint8)
    codes[:, 5] = 0x7e                                      # each row holds the maximum
    signs = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes = codes | signs
    for k in (-8, 0, 3):
        x = oracle.decode(oracle.E4M3, codes) * 2.0 ** k
        bits = oracle.encode(dt, x)
        assert np.array_equal(oracle.decode(dt, bits), x)   # exact in the 16-bit format
        q, s = oracle.quantize_e4m3_rows(dt, bits)
        assert np.all(s == np.float32(2.0 ** k))
        assert np.array_equal(q, codes)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.F16])
def test_quantize_row_maximum_and_error_bound(dt):
    x = inputs.normal((40, 256), 1.0, 99)
    x[3] *= 1e-3
    bits = inputs.to_bits(x, dt)
    xd = oracle.decode(dt, bits)
    q, s = oracle.quantize_e4m3_rows(dt, bits)
    amax = np.abs(xd).max(axis=1)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    dq = oracle.decode(oracle.E4M3, q) * s[:, None].astype(np.float64)
    # the largest magnitude of each row lands on +-448
    arg = np.abs(xd).argmax(axis=1)
    assert np.all((q[np.arange(40), arg] & 0x7f) == 0x7e)
    # three fraction bits: at most half a step, relative 2^-4, or 2^-10 * s below the normals
    bound = np.maximum(np.abs(xd) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(dq - xd) <= bound)


def test_quantize_zero_row_has_unit_scale():
    bits = np.zeros((2, 32), dtype=np.uint16)
    q, s = oracle.quantize_e4m3_rows(oracle.BF16, bits)
    assert np.all(s == 1.0) and not q.any()


def test_quantize_prune_compress_keeps_the_largest_codes():
    x = inputs.normal((8, 128), 1.0, 5)
    bits = inputs.to_bits(x, oracle.BF16)
    v, m, s = oracle.quantize_prune_compress(oracle.BF16, bits)
    q, s2 = oracle.quantize_e4m3_rows(oracle.BF16, bits)
    assert np.array_equal(s, s2)
    dense = oracle.decompress(oracle.E4M3, v, m, 128)
    qa = np.abs(oracle.decode(oracle.E4M3, q)).reshape(8, 32, 4)
    da = np.abs(oracle.decode(oracle.E4M3, dense)).reshape(8, 32, 4)
    # in every group the two kept magnitudes are the two largest of the codes
    assert np.array_equal(np.sort(da, axis=2)[:, :, 2:], np.sort(qa, axis=2)[:, :, 2:])


def test_quantize_decides_codes_in_fp32():
    """The quotient x / s is formed in fp32 before rounding to e4m3.  Search
    bf16 rows for elements whose fp32 quotient and exact quotient round to
    different codes, and check the oracle follows fp32 (numpy float32
    division, then torch's cast)."""
    all_bf16 = np.arange(0, 0x7f80, dtype=np.uint32).astype(np.uint16)    # finite positives
    vals = oracle.decode(oracle.BF16, all_bf16)
    found = 0
    for amax_bits in range(0x3f81, 0x3fff, 3):
        amax = oracle.decode(oracle.BF16, np.array([amax_bits], dtype=np.uint16))[0]
        s = np.float32(amax) / np.float32(448)
        cand = all_bf16[(vals > 0) & (vals < amax)]
        cv = oracle.decode(oracle.BF16, cand)
        q32 = (cv.astype(np.float32) / s).astype(np.float32)
        exact = cv / np.float64(s)
        c32, c64 = _torch_e4m3(q32), oracle.encode_e4m3(exact)
        diff = np.flatnonzero(c32 != c64)
        if len(diff) == 0:
            continue
        row = np.zeros((1, 32), dtype=np.uint16)
        row[0, 0] = amax_bits
        row[0, 1:1 + min(31, len(diff))] = cand[diff[:31]]
        q, sc = oracle.quantize_e4m3_rows(oracle.BF16, row)
        assert sc[0] == s
        xd = oracle.decode(oracle.BF16, row)[0].astype(np.float32)
        assert np.array_equal(q[0], _torch_e4m3((xd / s).astype(np.float32)))
        found += 1
        if found >= 3:
            break
    assert found >= 1, "no element found whose fp32 and fp64 quotients round apart"
