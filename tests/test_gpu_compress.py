"""GPU parity of prune+compress and decompress: bit-exact against the oracle
(values, metadata and the decompressed tensor), on every workload's operands
at full size and on edge cases (ties, signed zeros, NaN/Inf, ragged and
strided rows, misaligned buffers, K not a multiple of 32, empty inputs)."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import inputs
from tests._util import meta_host, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _check_compress(dt, bits, label):
    say("compress", label, bits.shape, "dt", dt)
    v_ref, m_ref = oracle.prune_compress(dt, bits)
    d = to_dev(bits, dt)
    v, m = sp.prune_compress(d)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(v, dt), v_ref), f"{label}: values differ"
    assert np.array_equal(meta_host(m), m_ref), f"{label}: metadata differ"
    back = sp.decompress(v, m, bits.shape[1])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(back, dt), oracle.decompress(dt, v_ref, m_ref, bits.shape[1])), \
        f"{label}: decompress differs"


@pytest.mark.parametrize("workload,s", [("tiny", 0), ("decode", 0), ("decode", 1), ("decode", 2),
                                        ("decode", 3), ("fp8", 0), ("fp8", 1), ("fp8", 2)])
def test_weights_full_size(workload, s):
    bits, _ = inputs.weight(workload, s)
    _check_compress(inputs.WORKLOADS[workload]["dtype"], bits, f"{workload} W{s}")


def test_online_activation_full_size():
    bits, _ = inputs.activation("online", 0, 0)
    _check_compress(oracle.BF16, bits, "online X")


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16, oracle.E4M3])
@pytest.mark.parametrize("rows,K", [(1, 16), (3, 32), (37, 104), (129, 1000), (64, 4096), (5, 4)])
def test_special_values_and_ragged_shapes(dt, rows, K):
    """Uniform random bit patterns: NaN, Inf, signed zeros, subnormals, ties."""
    bits = inputs.uniform_bits((rows, K), seed=rows * 7919 + K + dt, dt=dt)
    _check_compress(dt, bits, f"uniform bits {rows}x{K}")


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.E4M3])
def test_heavy_ties(dt):
    bits = inputs.integer_operand((256, 512), seed=5, dt=dt, lo=-1, hi=1)
    _check_compress(dt, bits, "ties from {-1,0,1}")


def test_strided_and_misaligned_source():
    dt = oracle.BF16
    full = inputs.uniform_bits((40, 200), seed=3, dt=dt)
    d = to_dev(full, dt)
    for col0, K in ((0, 192), (1, 196), (8, 100)):
        say("strided source", col0, K)
        view = d[:, col0:col0 + K]                          # row stride 200, start offset col0 elements
        v, m = sp.prune_compress(view)
        torch.cuda.synchronize()
        v_ref, m_ref = oracle.prune_compress(dt, full[:, col0:col0 + K])
        assert np.array_equal(to_host(v, dt), v_ref)
        assert np.array_equal(meta_host(m), m_ref)
        out = torch.zeros((40, 200), dtype=torch.bfloat16, device="cuda")
        sp.decompress(v, m, K, out=out[:, col0:col0 + K])
        torch.cuda.synchronize()
        ref = np.zeros((40, 200), np.uint16)
        ref[:, col0:col0 + K] = oracle.decompress(dt, v_ref, m_ref, K)
        assert np.array_equal(to_host(out, dt), ref)       # nothing outside the view was touched


def test_guard_bands_untouched():
    dt = oracle.BF16
    rows, K = 33, 96
    bits = inputs.uniform_bits((rows, K), seed=17, dt=dt)
    d = to_dev(bits, dt)
    guard = 1024
    vbuf = torch.full((rows * K // 2 + 2 * guard,), 0x5A5A, dtype=torch.int16, device="cuda")
    mbuf = torch.full((rows * 3 + 2 * guard,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
    v = vbuf[guard:guard + rows * K // 2].view(torch.bfloat16).view(rows, K // 2)
    m = mbuf[guard:guard + rows * 3].view(rows, 3)
    sp.prune_compress(d, values=v, meta=m)
    torch.cuda.synchronize()
    vb = vbuf.cpu().numpy()
    mb = mbuf.cpu().numpy()
    assert np.all(vb[:guard] == 0x5A5A) and np.all(vb[-guard:] == 0x5A5A)
    assert np.all(mb[:guard] == 0x3C3C3C3C) and np.all(mb[-guard:] == 0x3C3C3C3C)
    v_ref, m_ref = oracle.prune_compress(dt, bits)
    assert np.array_equal(to_host(v, dt), v_ref) and np.array_equal(meta_host(m), m_ref)


def test_empty_inputs():
    for shape in ((0, 64), (8, 0)):
        d = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        v, m = sp.prune_compress(d)
        assert v.shape == (shape[0], shape[1] // 2)


def test_deterministic_reruns():
    bits, _ = inputs.weight("decode", 0)
    d = to_dev(bits, oracle.BF16)
    v1, m1 = sp.prune_compress(d)
    v2, m2 = sp.prune_compress(d)
    torch.cuda.synchronize()
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)) and torch.equal(m1, m2)
