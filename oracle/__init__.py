"""CPU oracle for 2:4 semi-structured sparsity -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package.  The GPU library and its Python binding never import
it, and it imports nothing from them.

The arithmetic lives in ``sp24_oracle.c`` (plain C, fp64, built with gcc);
this module only marshals numpy arrays through ctypes.  Values are passed as
raw bit patterns: ``uint16`` for fp16/bf16, ``uint8`` for fp8 e4m3.

What is computed, and from which passages, is stated in the C file's header:
magnitude 2:4 pruning along K with ties to the lower index, packing into
half-width values plus one 4-bit (two 2-bit positions) nibble per group, the
inverse, and an fp64 GEMM on the decompressed operand.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

F16, BF16, E4M3, F32, I8 = 0, 1, 2, 3, 4
SPARSE_W, SPARSE_X = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def _load(path=None):
    """Loads (building it first if needed) the oracle library.  `path` loads a
    different build of the same source instead (used by the tests that plant
    mistakes in a copy of the oracle to show the pins catch them)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    if path is None:
        path = LIB_PATH
        if not os.path.exists(path):
            from . import build as _build
            _build.build()
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_e4m3.restype = ctypes.c_double
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_encode_f16.restype = ctypes.c_uint16
    lib.oracle_encode_f16.argtypes = [ctypes.c_double]
    lib.oracle_encode_bf16.restype = ctypes.c_uint16
    lib.oracle_encode_bf16.argtypes = [ctypes.c_double]
    lib.oracle_decode_array.restype = None
    lib.oracle_decode_array.argtypes = [i32, vp, i64, vp]
    lib.oracle_encode_array.restype = None
    lib.oracle_encode_array.argtypes = [i32, vp, i64, vp]
    lib.oracle_select_pair.restype = None
    lib.oracle_select_pair.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.oracle_meta_words_per_row.restype = i64
    lib.oracle_meta_words_per_row.argtypes = [i64]
    lib.oracle_prune_compress.restype = i32
    lib.oracle_prune_compress.argtypes = [i32, i64, i64, vp, i64, vp, vp]
    lib.oracle_decompress.restype = i32
    lib.oracle_decompress.argtypes = [i32, i64, i64, vp, vp, vp, i64]
    lib.oracle_encode_e4m3.restype = ctypes.c_uint8
    lib.oracle_encode_e4m3.argtypes = [ctypes.c_double]
    lib.oracle_quantize_e4m3_rows.restype = i32
    lib.oracle_quantize_e4m3_rows.argtypes = [i32, i64, i64, vp, i64, vp, vp]
    lib.oracle_encode_i8.restype = ctypes.c_int8
    lib.oracle_encode_i8.argtypes = [ctypes.c_float]
    lib.oracle_quantize_i8_rows.restype = i32
    lib.oracle_quantize_i8_rows.argtypes = [i32, i64, i64, vp, i64, vp, vp]
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
    lib.oracle_audit.restype = i32
    lib.oracle_audit.argtypes = [i64, vp, vp, vp, vp, vp, vp, ctypes.c_double, vp, vp]
    lib.oracle_num_threads.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [i32]
    _lib = lib
    return lib


class use_library:
    """Context manager: route every call to another build of the oracle
    source (a copy with a planted mistake, in the mutation tests)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bits_dtype(dt: int):
    return {F16: np.uint16, BF16: np.uint16, E4M3: np.uint8, F32: np.uint32, I8: np.uint8}[dt]


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Worker threads of later oracle calls (for timing the CPU baseline)."""
    _load().oracle_set_num_threads(int(n))


def decode(dt: int, bits: np.ndarray) -> np.ndarray:
    """Bit patterns of format `dt` -> float64, from the format definitions."""
    bits = np.ascontiguousarray(bits, dtype=_bits_dtype(dt))
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_decode_array(dt, _ptr(bits), bits.size, _ptr(out))
    return out


def encode(dt: int, x: np.ndarray) -> np.ndarray:
    """float64 -> fp16/bf16 bit patterns, round to nearest even."""
    assert dt in (F16, BF16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_encode_array(dt, _ptr(x), x.size, _ptr(out))
    return out


def select_pair(keys) -> tuple[int, int]:
    """The kept positions (p0 < p1) of one group given 4 magnitude keys."""
    k = np.ascontiguousarray(keys, dtype=np.uint32)
    assert k.shape == (4,)
    p0, p1 = ctypes.c_int(), ctypes.c_int()
    _load().oracle_select_pair(_ptr(k), ctypes.byref(p0), ctypes.byref(p1))
    return p0.value, p1.value


def meta_words_per_row(K: int) -> int:
    return (K + 31) // 32


def prune_compress(dt: int, src: np.ndarray):
    """Dense rows x K bit patterns -> (values rows x K/2, meta rows x ceil(K/32) uint32)."""
    src = np.ascontiguousarray(src, dtype=_bits_dtype(dt))
    rows, K = src.shape
    values = np.empty((rows, K // 2), dtype=src.dtype)
    meta = np.empty((rows, meta_words_per_row(K)), dtype=np.uint32)
    rc = _load().oracle_prune_compress(dt, rows, K, _ptr(src), K, _ptr(values), _ptr(meta))
    if rc != 0:
        raise ValueError(f"oracle_prune_compress rejected dt={dt} shape={src.shape}")
    return values, meta


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """fp64 values -> OCP e4m3fn codes, round to nearest even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    f = _load().oracle_encode_e4m3
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def quantize_e4m3_rows(dt: int, src: np.ndarray):
    """16-bit rows x K bit patterns -> (e4m3 codes rows x K, fp32 scale per row)."""
    src = np.ascontiguousarray(src, dtype=_bits_dtype(dt))
    rows, K = src.shape
    q = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    rc = _load().oracle_quantize_e4m3_rows(dt, rows, K, _ptr(src), K, _ptr(q), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_quantize_e4m3_rows rejected dt={dt} shape={src.shape}")
    return q, scales


def quantize_prune_compress(dt: int, src: np.ndarray):
    """The fused online fp8 path: per-row quantization to e4m3, then 2:4 prune
    and compress of the codes -> (values rows x K/2, meta, scales)."""
    q, scales = quantize_e4m3_rows(dt, src)
    values, meta = prune_compress(E4M3, q)
    return values, meta, scales


def encode_i8(t: float) -> int:
    """The int8 code of an fp32 quotient (nearest, ties to even, saturated to +-127; NaN -> 0)."""
    return int(_load().oracle_encode_i8(float(t)))


def quantize_i8_rows(dt: int, src: np.ndarray):
    """16-bit rows x K bit patterns -> (int8 codes rows x K as uint8 bytes, fp32 scale per row)."""
    src = np.ascontiguousarray(src, dtype=_bits_dtype(dt))
    rows, K = src.shape
    q = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    rc = _load().oracle_quantize_i8_rows(dt, rows, K, _ptr(src), K, _ptr(q), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_quantize_i8_rows rejected dt={dt} shape={src.shape}")
    return q, scales


def quantize_i8_prune_compress(dt: int, src: np.ndarray):
    """The fused online int8 path: per-row quantization to int8, then 2:4 prune
    and compress of the codes -> (values rows x K/2, meta, scales)."""
    q, scales = quantize_i8_rows(dt, src)
    values, meta = prune_compress(I8, q)
    return values, meta, scales


def decompress(dt: int, values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    values = np.ascontiguousarray(values, dtype=_bits_dtype(dt))
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    rows = values.shape[0]
    assert values.shape == (rows, K // 2) and meta.shape == (rows, meta_words_per_row(K))
    dst = np.empty((rows, K), dtype=values.dtype)
    rc = _load().oracle_decompress(dt, rows, K, _ptr(values), _ptr(meta), _ptr(dst), K)
    if rc != 0:
        raise ValueError("oracle_decompress rejected its arguments")
    return dst


def prune(dt: int, src: np.ndarray) -> np.ndarray:
    """The pruned dense tensor: decompress(compress(src))."""
    v, m = prune_compress(dt, src)
    return decompress(dt, v, m, src.shape[1])


def gemm(dt: int, M: int, N: int, K: int, *, x=None, x_vals=None, x_meta=None,
         w=None, w_vals=None, w_meta=None, scale_x=None, scale_w=None, mrows=None):
    """R = X * W^T in fp64 for the listed X rows (all rows if mrows is None).

    Exactly one of x / (x_vals, x_meta) and one of w / (w_vals, w_meta) is
    given; a compressed operand is decompressed first.
    """
    bd = _bits_dtype(dt)
    c = lambda a, d: None if a is None else np.ascontiguousarray(a, dtype=d)
    x, x_vals, w, w_vals = c(x, bd), c(x_vals, bd), c(w, bd), c(w_vals, bd)
    x_meta, w_meta = c(x_meta, np.uint32), c(w_meta, np.uint32)
    scale_x, scale_w = c(scale_x, np.float32), c(scale_w, np.float32)
    if mrows is None:
        mrows = np.arange(M, dtype=np.int64)
    mrows = np.ascontiguousarray(mrows, dtype=np.int64)
    if x is not None:
        assert x.shape == (M, K)
    else:
        assert x_vals.shape == (M, K // 2) and x_meta.shape == (M, meta_words_per_row(K))
    if w is not None:
        assert w.shape == (N, K)
    else:
        assert w_vals.shape == (N, K // 2) and w_meta.shape == (N, meta_words_per_row(K))
    if scale_x is not None:
        assert scale_x.shape == (M,)
    if scale_w is not None:
        assert scale_w.shape == (N,)
    R = np.empty((len(mrows), N), dtype=np.float64)
    rc = _load().oracle_gemm(dt, M, N, K, _ptr(x), _ptr(x_vals), _ptr(x_meta),
                             _ptr(w), _ptr(w_vals), _ptr(w_meta),
                             _ptr(scale_x), _ptr(scale_w), _ptr(mrows), len(mrows), _ptr(R))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return R


def hybrid_gemm(dt: int, M: int, NS: int, ND: int, K: int, *, x, ws_vals=None, ws_meta=None, wd=None,
                scale_x=None, scale_w=None):
    """The row-split hybrid ("Production 2:4 Structured Sparsity for LLMs",
    "Dense Fallback and Hybrid Sparsity Design"): R = X [Ws | Wd]^T, the first
    NS output columns from the 2:4 rows (decompressed), the next ND from the
    dense rows; each block is the plain product of gemm()."""
    R = np.zeros((M, NS + ND), dtype=np.float64)
    sw = None if scale_w is None else np.asarray(scale_w, dtype=np.float32)
    if NS > 0:
        R[:, :NS] = gemm(dt, M, NS, K, x=x, w_vals=ws_vals, w_meta=ws_meta, scale_x=scale_x,
                         scale_w=None if sw is None else sw[:NS])
    if ND > 0:
        R[:, NS:] = gemm(dt, M, ND, K, x=x, w=wd, scale_x=scale_x, scale_w=None if sw is None else sw[NS:])
    return R


def ksplit_gemm(dt: int, M: int, N: int, KS: int, K: int, *, x, ws_vals, ws_meta, wd, scale_x=None,
                scale_w=None, mrows=None):
    """The K-split hybrid ("Production 2:4 Structured Sparsity for LLMs",
    "Dense Fallback and Hybrid Sparsity Design"; the SlideSparse page's
    Spense abstract: each weight split into a 2:4 region and a dense region):
    columns [0, KS) of every weight row are 2:4 (given compressed), columns
    [KS, K) dense (wd, N x (K - KS)).  The weight is the two ranges side by
    side along K, the 2:4 range decompressed; R = X W^T over that weight, the
    plain product of gemm()."""
    KD = K - KS
    assert 0 <= KS <= K
    ws = decompress(dt, ws_vals, ws_meta, KS) if KS > 0 else np.zeros((N, 0), dtype=_bits_dtype(dt))
    wd = np.zeros((N, 0), dtype=_bits_dtype(dt)) if KD == 0 else np.ascontiguousarray(wd, dtype=_bits_dtype(dt))
    assert ws.shape == (N, KS) and wd.shape == (N, KD)
    w = np.ascontiguousarray(np.concatenate([ws, wd], axis=1))
    return gemm(dt, M, N, K, x=x, w=w, scale_x=scale_x, scale_w=scale_w, mrows=mrows)


def audit_metrics(records, counts, other_time_us: float = 0.0) -> dict:
    """Manifest metrics over layer records (dicts with eligible, selected
    ("sparse" / "dense"), t_sparse_us, t_compress_us, t_dense_us), record i
    standing for counts[i] layers."""
    n = len(records)
    el = np.array([int(bool(r["eligible"])) for r in records] or [0], dtype=np.int32)
    sel = np.array([int(r["selected"] == "sparse") for r in records] or [0], dtype=np.int32)
    ts = np.array([float(r["t_sparse_us"]) for r in records] or [0.0])
    tc = np.array([float(r["t_compress_us"]) for r in records] or [0.0])
    td = np.array([float(r["t_dense_us"]) for r in records] or [0.0])
    cnt = np.array(list(counts) or [0], dtype=np.int64)
    co = np.zeros(4, dtype=np.int64)
    ro = np.zeros(5)
    st = _load().oracle_audit(n, _ptr(el), _ptr(sel), _ptr(ts), _ptr(tc), _ptr(td), _ptr(cnt),
                              float(other_time_us), _ptr(co), _ptr(ro))
    if st != 0:
        raise ValueError("oracle_audit rejected its arguments")
    return {"candidate_layers": int(co[0]), "eligible_layers": int(co[1]), "sparse_selected_layers": int(co[2]),
            "dense_fallback_layers": int(co[3]), "eligibility_ratio": float(ro[0]),
            "sparse_selection_ratio": float(ro[1]), "sparse_gpu_time_us": float(ro[2]),
            "total_gpu_time_us": float(ro[3]), "sparse_gpu_time_coverage": float(ro[4])}


def relative_error(Y: np.ndarray, R: np.ndarray) -> float:
    """max |Y - R| / max(|R|, rms(R)): the GEMM parity measure.

    The denominator is floored at the root-mean-square of R so that the few
    outputs that sit near zero by cancellation do not turn ordinary fp32
    accumulation error into a large relative error.
    """
    Y = np.asarray(Y, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    if R.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(R * R)))
    denom = np.maximum(np.abs(R), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(Y - R) / denom))
