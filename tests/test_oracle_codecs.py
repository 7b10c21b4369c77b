"""Pins the oracle's number-format codecs to torch's CPU casts (a library
routine), exhaustively for every 16-bit and 8-bit pattern."""
import numpy as np
import torch

import oracle


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_decode_every_f16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    assert _same(oracle.decode(oracle.F16, bits), ref)


def test_decode_every_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(oracle.decode(oracle.BF16, bits), ref)


def test_decode_every_e4m3_pattern():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode(oracle.E4M3, bits)
    assert _same(got, ref)
    # format facts: largest finite 448, smallest subnormal 2^-9, no infinities
    assert np.nanmax(got) == 448.0
    assert np.nanmin(np.abs(got[got != 0])) == 2.0 ** -9
    assert not np.any(np.isinf(got))
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_decode_f32_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0, 0x80000000, 1, 0x7F800000, 0xFF800000, 0x7FC00000, 0x007FFFFF, 0x3F800000]
    assert _same(oracle.decode(oracle.F32, bits), bits.view(np.float32).astype(np.float64))


def _fp32_sample(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(-149, 128, n)
    sign = rng.choice([-1.0, 1.0], n)
    x = (sign * np.ldexp(mant, exp)).astype(np.float32)   # every value exact in fp32
    return x


def _halfway(dt):
    """Exact midpoints between consecutive finite values of the format."""
    bits = np.arange(0, 0x7C00 if dt == oracle.F16 else 0x7F80, dtype=np.uint16)
    v = oracle.decode(dt, bits)
    mids = (v[:-1] + v[1:]) / 2.0           # exact in fp64, and in fp32
    return np.concatenate([mids, -mids]).astype(np.float32)


def _check_encoder(dt, tdt):
    x = np.concatenate([_fp32_sample(1_000_000, 1 + dt), _halfway(dt),
                        np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.996, 65520.0,
                                  3.3895314e38, 3.40e38], dtype=np.float32)])
    ref = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode(dt, x.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"first mismatches: {[(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]}"


def test_encode_f16_rne_matches_torch():
    _check_encoder(oracle.F16, torch.float16)


def test_encode_bf16_rne_matches_torch():
    _check_encoder(oracle.BF16, torch.bfloat16)


def test_encode_decode_roundtrip():
    for dt in (oracle.F16, oracle.BF16):
        bits = np.arange(65536, dtype=np.uint16)
        v = oracle.decode(dt, bits)
        keep = ~np.isnan(v)
        assert np.array_equal(oracle.encode(dt, v[keep]), bits[keep])
