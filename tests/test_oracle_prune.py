"""Pins the oracle's 2:4 prune / compress / decompress to facts the pages and
the mathematics fix: the pages' worked example, brute force over the six
possible pairs, a second brute force on decoded magnitudes, the pages'
top-2 library recipe on tie-free data, and the format's invariants and byte
accounting."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from semi_structured_sparse_sp24_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAIRS = list(itertools.combinations(range(4), 2))          # the six possible kept pairs
LEGAL_NIBBLES = {p0 | (p1 << 2) for p0, p1 in PAIRS}


def _golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                rows[k] = v
    return rows


def _nibbles(meta, K):
    g = np.arange(K // 4)
    return (meta[:, g // 8] >> (4 * (g % 8)).astype(np.uint32)) & 0xF


# ---------------------------------------------------------------- worked example

@pytest.mark.parametrize("dt,tdt", [(oracle.F16, torch.float16), (oracle.BF16, torch.bfloat16)])
def test_worked_example(dt, tdt):
    g = _golden("worked_example.txt")
    dense = np.array([float(v) for v in g["dense"]], dtype=np.float32)
    pruned = np.array([float(v) for v in g["pruned"]])
    bits = torch.from_numpy(dense).to(tdt).view(torch.int16).numpy().view(np.uint16)[None, :]
    vals, meta = oracle.prune_compress(dt, bits)
    assert meta.shape == (1, 1)
    assert int(meta[0, 0]) == 0xC                         # positions 0 and 3
    assert list(vals[0]) == [bits[0, 0], bits[0, 3]]      # kept values, bit for bit
    back = oracle.decode(dt, oracle.decompress(dt, vals, meta, 4))[0]
    assert np.allclose(back, pruned, atol=5e-3)
    assert back[1] == 0.0 and back[2] == 0.0 and not np.signbit(back[1]) and not np.signbit(back[2])


# ---------------------------------------------------------------- brute force

def _brute_force_pair(keys):
    """The unique pair (i, j) such that every kept key >= every dropped key and
    a dropped key equal to a kept key only sits at a higher index."""
    valid = []
    for i, j in PAIRS:
        kept, dropped = (i, j), [d for d in range(4) if d not in (i, j)]
        ok = all(keys[k] >= keys[d] for k in kept for d in dropped)
        ok = ok and all(not (keys[k] == keys[d] and d < k) for k in kept for d in dropped)
        if ok:
            valid.append((i, j))
    assert len(valid) == 1, (keys, valid)
    return valid[0]


@pytest.mark.parametrize("alphabet", [4, 8])
def test_select_pair_exhaustive(alphabet):
    for keys in itertools.product(range(alphabet), repeat=4):
        assert oracle.select_pair(keys) == _brute_force_pair(keys), keys


def test_select_pair_random_wide_keys():
    rng = np.random.default_rng(5)
    for keys in rng.integers(0, 0x8000, size=(20000, 4)):
        assert oracle.select_pair(keys) == _brute_force_pair(list(keys))


def _fp64_brute_force(dec_row):
    """Second brute force on decoded values: the pair with the largest
    |a| + |b|, the lexicographically smallest on equal sums.  For non-NaN
    inputs whose sums are exact in fp64, a pair reaching the maximum must hold
    the two largest magnitudes, so this is the same selection."""
    best = None
    for i, j in PAIRS:
        s = abs(dec_row[i]) + abs(dec_row[j])
        if best is None or s > best[0]:
            best = (s, (i, j))
    return best[1]


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16, oracle.E4M3])
def test_compress_matches_fp64_brute_force(dt):
    # Heavy ties: values drawn from a small set (with both signed zeros).
    rng = np.random.default_rng(11 + dt)
    g = torch.Generator("cpu").manual_seed(3 + dt)
    rows, K = 64, 256
    smooth = torch.randn(rows, K, generator=g) * 2.0
    coarse = torch.from_numpy(rng.choice([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], size=(rows, K)).astype(np.float32))
    t = torch.where(torch.from_numpy(rng.random((rows, K)) < 0.5), smooth, coarse)
    if dt == oracle.E4M3:
        t = t.clamp(-448, 448)
    bits = inputs.to_bits(t, dt)
    vals, meta = oracle.prune_compress(dt, bits)
    nib = _nibbles(meta, K)
    dec = oracle.decode(dt, bits)
    for r in range(rows):
        for gi in range(K // 4):
            p = _fp64_brute_force(dec[r, 4 * gi:4 * gi + 4])
            assert nib[r, gi] == (p[0] | (p[1] << 2)), (r, gi, dec[r, 4 * gi:4 * gi + 4])


def test_compress_matches_topk_recipe_on_tie_free_data():
    """The pages' PyTorch recipe: group-wise top-2 magnitudes, scatter a mask."""
    w = inputs.normal((512, 1024), 0.02, seed=77)
    bits = inputs.to_bits(w, oracle.BF16)
    wq = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    groups = wq.abs().reshape(-1, 4)
    tie_free = torch.tensor([len(set(row.tolist())) == 4 for row in groups])
    mask = torch.zeros_like(groups, dtype=torch.bool)
    mask.scatter_(1, groups.topk(2, dim=1).indices, True)
    ref = torch.where(mask, wq.reshape(-1, 4), torch.zeros_like(groups))
    got = torch.from_numpy(oracle.decode(oracle.BF16, oracle.prune(oracle.BF16, bits))).reshape(-1, 4)
    assert tie_free.float().mean() > 0.9
    assert torch.equal(got[tie_free].float(), ref[tie_free])


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16, oracle.E4M3])
@pytest.mark.parametrize("K", [4, 28, 32, 100, 256])
def test_format_invariants(dt, K):
    rows = 37
    bits = inputs.uniform_bits((rows, K), seed=1000 + K + dt, dt=dt)
    vals, meta = oracle.prune_compress(dt, bits)
    assert vals.shape == (rows, K // 2) and meta.shape == (rows, math.ceil(K / 32))
    nib = _nibbles(meta, K)
    assert set(np.unique(nib)) <= LEGAL_NIBBLES
    # unused high nibbles of the last word are zero
    if K % 32:
        used = (K // 4) % 8
        assert np.all(meta[:, -1] >> np.uint32(4 * used) == 0)
    dense = oracle.decompress(dt, vals, meta, K)
    mask = 0x7F if dt == oracle.E4M3 else 0x7FFF
    for r in range(rows):
        for g in range(K // 4):
            p0, p1 = nib[r, g] & 3, nib[r, g] >> 2
            grp = dense[r, 4 * g:4 * g + 4]
            src = bits[r, 4 * g:4 * g + 4]
            # kept values are the input bits, in ascending position order
            assert vals[r, 2 * g] == src[p0] and vals[r, 2 * g + 1] == src[p1]
            assert grp[p0] == src[p0] and grp[p1] == src[p1]
            # dropped positions are +0.0, and no dropped magnitude beats a kept one
            for d in set(range(4)) - {p0, p1}:
                assert grp[d] == 0
                assert (src[d] & mask) <= min(src[p0] & mask, src[p1] & mask)
    # compress(decompress(c)) == c  and prune is idempotent
    v2, m2 = oracle.prune_compress(dt, dense)
    assert np.array_equal(v2, vals) and np.array_equal(m2, meta)


def test_exactly_two_kept_slots_and_nonzero_count():
    """Every group keeps exactly two slots; the pruned view has exactly two
    nonzeros unless the input group itself had fewer."""
    bits = inputs.weight("tiny", 0)[0]
    dec_in = oracle.decode(oracle.F16, bits).reshape(-1, 4)
    dec_out = oracle.decode(oracle.F16, oracle.prune(oracle.F16, bits)).reshape(-1, 4)
    nnz_in = (dec_in != 0).sum(1)
    nnz_out = (dec_out != 0).sum(1)
    assert np.all(nnz_out == np.minimum(nnz_in, 2))


def test_storage_accounting_matches_pages():
    st = _golden("storage_fp16.txt")
    pt = _golden("patterns.txt")
    rows, K = 8, 256
    bits = inputs.uniform_bits((rows, K), seed=9, dt=oracle.F16)
    vals, meta = oracle.prune_compress(oracle.F16, bits)
    groups = rows * K // 4
    bits_per_group_sparse = (vals.nbytes + meta.nbytes) * 8 / groups
    bits_per_group_dense = bits.nbytes * 8 / groups
    assert bits_per_group_dense == int(st["dense"][0])
    assert bits_per_group_sparse == int(st["sp24"][0])
    assert round(100 * bits_per_group_sparse / bits_per_group_dense) == int(st["sp24"][1])
    # metadata: 1 bit per element; six patterns, ideal log2(6)/4 bits
    assert meta.nbytes * 8 / (rows * K) == int(pt["hardware_bits_per_element"][0])
    assert len(LEGAL_NIBBLES) == int(pt["patterns"][0])
    assert round(math.log2(len(LEGAL_NIBBLES)) / 4, 2) == float(pt["ideal_bits_per_element"][0])
    # compression ratio 2k/(k+2) for k-bit values (k = 16 here, and 8 for e4m3)
    for dt, k in ((oracle.F16, 16), (oracle.E4M3, 8)):
        b = inputs.uniform_bits((rows, K), seed=10, dt=dt)
        v, m = oracle.prune_compress(dt, b)
        assert b.nbytes / (v.nbytes + m.nbytes) == pytest.approx(2 * k / (k + 2))


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.prune_compress(oracle.F16, np.zeros((2, 6), np.uint16))
    with pytest.raises(ValueError):
        oracle.prune_compress(oracle.F32, np.zeros((2, 8), np.uint32))


def test_empty_inputs():
    v, m = oracle.prune_compress(oracle.BF16, np.zeros((0, 64), np.uint16))
    assert v.shape == (0, 32) and m.shape == (0, 2)
    v, m = oracle.prune_compress(oracle.BF16, np.zeros((3, 0), np.uint16))
    assert v.shape == (3, 0) and m.shape == (3, 0)
