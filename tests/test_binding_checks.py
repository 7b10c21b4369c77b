"""The Python binding rejects every tensor that does not match M, N and K
(shape, row stride, contiguity, dtype, device) before anything reaches the
library: the kernels size their buffer descriptors and grids from the sizes
alone, so a mismatched tensor would otherwise be read or written out of
bounds.  Runs on the CPU: the library is replaced by a stub that fails the
test if any entry point is called."""
import pytest
import torch

import semi_structured_sparse_sp24_amd as sp


class _NoLaunch:
    def __getattr__(self, name):
        raise AssertionError(f"library entry point {name} reached despite bad arguments")


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    monkeypatch.setattr(sp, "lib", lambda: _NoLaunch())


BF, E4 = torch.bfloat16, torch.float8_e4m3fn
M, N, K = 8, 64, 128


def _good():
    """Operands of a weight-compressed GEMM of M x N x K, all well formed (on the CPU)."""
    return dict(v=torch.zeros((N, K // 2), dtype=BF), m=torch.zeros((N, K // 32), dtype=torch.int32),
                x=torch.zeros((M, K), dtype=BF), out=torch.zeros((M, N), dtype=BF),
                sx=torch.ones(M), sw=torch.ones(N))


def _gemm(**kw):
    a = _good()
    a.update(kw)
    return sp.sp24_gemm(sp.SPARSE_W, a["v"], a["m"], a["x"], M, N, K, scale_x=a["sx"], scale_w=a["sw"],
                        out=a["out"])


@pytest.mark.parametrize("bad", [
    dict(v=torch.zeros((N, K // 2 - 8), dtype=BF)),                 # values too short for K
    dict(v=torch.zeros((N - 1, K // 2), dtype=BF)),                 # values for fewer rows
    dict(m=torch.zeros((N, K // 32 - 1), dtype=torch.int32)),       # metadata too short
    dict(x=torch.zeros((M, K + 64), dtype=BF)),                     # a different K
    dict(x=torch.zeros((M + 1, K), dtype=BF)),                      # a different M
    dict(x=torch.zeros((K, M), dtype=BF).t()),                      # transposed view
    dict(x=torch.zeros((M, 2 * K), dtype=BF)[:, :K]),               # padded rows
    dict(out=torch.zeros((M, N + 8), dtype=BF)),                    # output of another shape
    dict(out=torch.zeros((N, M), dtype=BF).t()),                    # transposed output
    dict(sx=torch.ones(M + 1)),                                     # scale of another length
    dict(sw=torch.ones(2 * N)[::2]),                                # strided scale
])
def test_sparse_gemm_shape_and_stride_mismatches_raise(bad):
    with pytest.raises(ValueError):
        _gemm(**bad)


@pytest.mark.parametrize("bad", [
    dict(v=torch.zeros((N, K // 2), dtype=torch.float16)),          # values of another dtype
    dict(m=torch.zeros((N, K // 32), dtype=torch.float32)),         # metadata not int32
    dict(sw=torch.ones(N, dtype=torch.float64)),
])
def test_sparse_gemm_dtype_mismatches_raise(bad):
    with pytest.raises((TypeError, ValueError)):
        _gemm(**bad)


def test_well_formed_host_tensors_are_refused_for_their_device():
    with pytest.raises(ValueError, match="GPU"):
        _gemm()


def test_activation_compressed_gemm_checks_rows_of_x():
    g = _good()
    xv = torch.zeros((M, K // 2), dtype=BF)
    xm = torch.zeros((M, K // 32), dtype=torch.int32)
    w = torch.zeros((N, K), dtype=BF)
    with pytest.raises(ValueError, match="GPU"):
        sp.sp24_gemm(sp.SPARSE_X, xv, xm, w, M, N, K, out=g["out"])
    with pytest.raises(ValueError):   # the weight's compressed form where X's belongs
        sp.sp24_gemm(sp.SPARSE_X, g["v"], g["m"], w, M, N, K, out=g["out"])
    with pytest.raises(ValueError):
        sp.sp24_gemm(7, xv, xm, w, M, N, K)


def test_dense_gemm_checks():
    x, w = torch.zeros((M, K), dtype=BF), torch.zeros((N, K), dtype=BF)
    with pytest.raises(TypeError):
        sp.dense_gemm(x, w.to(torch.float16))
    with pytest.raises(ValueError):
        sp.dense_gemm(x, torch.zeros((K, N), dtype=BF).t())
    with pytest.raises(ValueError):
        sp.dense_gemm(x, w, out=torch.zeros((M, N - 1), dtype=BF))
    with pytest.raises(ValueError):
        sp.dense_gemm(x, w, scale_x=torch.ones(M - 1))
    with pytest.raises(ValueError, match="GPU"):
        sp.dense_gemm(x, w, out=torch.zeros((M, N), dtype=BF))


def test_prune_compress_and_decompress_checks():
    d = torch.zeros((N, K), dtype=BF)
    with pytest.raises(ValueError):
        sp.prune_compress(d, values=torch.zeros((N, K // 4), dtype=BF))
    with pytest.raises(TypeError):
        sp.prune_compress(d, values=torch.zeros((N, K // 2), dtype=torch.float16))
    with pytest.raises(ValueError):
        sp.prune_compress(torch.zeros((K, N), dtype=BF).t())            # K not contiguous
    with pytest.raises(ValueError, match="GPU"):
        sp.prune_compress(torch.zeros((N, 2 * K), dtype=BF)[:, :K])     # a row stride above K is fine
    v, m = torch.zeros((N, K // 2), dtype=BF), torch.zeros((N, K // 32), dtype=torch.int32)
    with pytest.raises(ValueError):
        sp.decompress(v, m, 2 * K)                                      # K does not match the values
    with pytest.raises(ValueError):
        sp.decompress(v, m, K, out=torch.zeros((N, K - 4), dtype=BF))
    with pytest.raises(TypeError):
        sp.decompress(v, m, K, out=torch.zeros((N, K), dtype=torch.float16))


def test_quantizer_checks():
    x = torch.zeros((M, K), dtype=BF)
    with pytest.raises(TypeError):
        sp.quantize_prune_compress(x, values=torch.zeros((M, K // 2), dtype=BF))
    with pytest.raises(ValueError):
        sp.quantize_prune_compress(x, scales=torch.ones(M + 1))
    with pytest.raises(ValueError):
        sp.quantize_e4m3(x, out=torch.zeros((M, K // 2), dtype=E4))
    with pytest.raises(TypeError):
        sp.quantize_i8_prune_compress(x, values=torch.zeros((M, K // 2), dtype=E4))
    with pytest.raises(ValueError):
        sp.quantize_i8_prune_compress(x, meta=torch.zeros((M, K // 32 + 1), dtype=torch.int32))
    with pytest.raises(TypeError):
        sp.quantize_i8(x, out=torch.zeros((M, K), dtype=torch.uint8))
    with pytest.raises(ValueError):
        sp.quantize_i8(x.t())


def test_hybrid_checks():
    NS, ND = 48, 16
    x = torch.zeros((M, K), dtype=BF)
    v, m = torch.zeros((NS, K // 2), dtype=BF), torch.zeros((NS, K // 32), dtype=torch.int32)
    wd = torch.zeros((ND, K), dtype=BF)
    with pytest.raises(ValueError):
        sp.hybrid_gemm(v, m, wd, x, NS + 8, ND)
    with pytest.raises(ValueError):
        sp.hybrid_gemm(v, m, torch.zeros((ND, K + 32), dtype=BF), x, NS, ND)
    with pytest.raises(ValueError):
        sp.hybrid_gemm(v, m, wd, x, NS, ND, scale_w=torch.ones(NS))
    with pytest.raises(ValueError, match="GPU"):
        sp.hybrid_gemm(v, m, wd, x, NS, ND)


def test_select_tactic_checks():
    g = _good()
    wp = torch.zeros((N, K), dtype=BF)
    with pytest.raises(ValueError):
        sp.select_tactic(sp.SPARSE_W, g["v"], g["m"], g["x"], torch.zeros((N, K // 2), dtype=BF), M, N, K)
    with pytest.raises(ValueError):
        sp.select_tactic(sp.SPARSE_W, g["v"], g["m"], g["x"], wp, M, N, K,
                         y_scratch=torch.zeros((M, N // 2), dtype=BF))
    with pytest.raises(ValueError, match="GPU"):
        sp.select_tactic(sp.SPARSE_W, g["v"], g["m"], g["x"], wp, M, N, K, y_scratch=g["out"])
