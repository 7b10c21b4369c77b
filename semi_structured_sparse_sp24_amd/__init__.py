"""2:4 semi-structured sparse GEMM for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libsp24.so (C ABI in include/sp24.h).  Every step
of the path runs in the library's HIP kernels; this module only checks
Python-level arguments, allocates outputs with torch (device memory) and
passes raw pointers plus torch's current HIP stream.  There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

  prune_compress(w)            -> (values, meta)       magnitude 2:4 along K
  decompress(values, meta, K)  -> dense pruned tensor
  sp24_gemm(...)               -> Y = X W^T with W (or X) compressed
  dense_gemm(x, w, ...)        -> Y = X W^T, the dense baseline
  select_tactic(...)           -> per-shape sparse-or-dense record
  tactic_decide(...)           -> the decision rule on given timings (host only)
  gemm_kernel(...)             -> name of the kernel a GEMM call would launch (host only)
  quantize_prune_compress(x)   -> (values e4m3, meta, scales): fused online fp8 path
  quantize_e4m3(x)             -> (codes e4m3, scales): the dense side's quantization
  hybrid_gemm(...)             -> Y = X [Ws | Wd]^T, Ws compressed and Wd dense rows, one launch
  audit_aggregate(...)         -> layer counts, ratios and Sparse GPU-Time Coverage (host only)
"""
from __future__ import annotations

import ctypes
import os

import torch

F16, BF16, E4M3, F32, I8 = 0, 1, 2, 3, 4
SPARSE_W, SPARSE_X = 0, 1
STATUS = {0: "SP24_OK", 1: "SP24_E_NULL", 2: "SP24_E_SHAPE", 3: "SP24_E_DTYPE", 4: "SP24_E_ALIGN",
          5: "SP24_E_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsp24.so")

# Every function the header declares, with its ctypes signature.
_vp, _i64, _i32, _dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double


class Tactic(ctypes.Structure):
    _fields_ = [("eligible", ctypes.c_int), ("selected", ctypes.c_int),
                ("t_sparse_us", ctypes.c_double), ("t_compress_us", ctypes.c_double),
                ("t_dense_us", ctypes.c_double), ("ratio", ctypes.c_double),
                ("reason", ctypes.c_char * 96), ("kernel", ctypes.c_char * 64)]

    def as_dict(self):
        return {"eligible": bool(self.eligible), "selected": "sparse" if self.selected else "dense",
                "t_sparse_us": self.t_sparse_us, "t_compress_us": self.t_compress_us,
                "t_dense_us": self.t_dense_us, "ratio": self.ratio,
                "reason": self.reason.decode(), "kernel": self.kernel.decode()}


class AuditMetrics(ctypes.Structure):
    _fields_ = [("candidate_layers", ctypes.c_int64), ("eligible_layers", ctypes.c_int64),
                ("sparse_selected_layers", ctypes.c_int64), ("dense_fallback_layers", ctypes.c_int64),
                ("eligibility_ratio", ctypes.c_double), ("sparse_selection_ratio", ctypes.c_double),
                ("sparse_gpu_time_us", ctypes.c_double), ("total_gpu_time_us", ctypes.c_double),
                ("sparse_gpu_time_coverage", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


SIGNATURES = {
    "sp24_status_str": (ctypes.c_char_p, [_i32]),
    "sp24_version": (ctypes.c_char_p, []),
    "sp24_meta_words_per_row": (_i64, [_i64]),
    "sp24_prune_compress": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "sp24_decompress": (_i32, [_i32, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "sp24_gemm": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "dense_gemm": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sp24_select_tactic": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _i32, _i32, _vp, ctypes.POINTER(Tactic)]),
    "sp24_tactic_decide": (_i32, [_i32, ctypes.POINTER(_dbl), _i32, ctypes.POINTER(_dbl), _i32,
                                  ctypes.POINTER(Tactic)]),
    "sp24_gemm_kernel": (ctypes.c_char_p, [_i32, _i32, _i32, _i32, _i64, _i64, _i64]),
    "sp24_hybrid_gemm": (_i32, [_i32, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sp24_hybrid_kernel": (ctypes.c_char_p, [_i32, _i32, _i64, _i64, _i64, _i64]),
    "sp24_audit_aggregate": (_i32, [ctypes.POINTER(Tactic), ctypes.POINTER(_i64), _i64, _dbl,
                                    ctypes.POINTER(AuditMetrics)]),
    "sp24_quantize_prune_compress": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp]),
    "sp24_quantize_e4m3": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
}

_lib = None


class Sp24Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}")


def lib():
    """The loaded libsp24.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m semi_structured_sparse_sp24_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(fn, st):
    if st != 0:
        raise Sp24Error(fn, st)


DTYPE_CODE = {torch.float16: F16, torch.bfloat16: BF16, torch.float8_e4m3fn: E4M3, torch.float32: F32,
              torch.int8: I8}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}


def _code(t: torch.Tensor) -> int:
    if t.dtype not in DTYPE_CODE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return DTYPE_CODE[t.dtype]


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def meta_words_per_row(K: int) -> int:
    return int(lib().sp24_meta_words_per_row(K))


def prune_compress(dense: torch.Tensor, values=None, meta=None):
    """Magnitude 2:4 along the last axis: (values rows x K/2, meta rows x ceil(K/32) int32)."""
    assert dense.dim() == 2 and dense.is_cuda and dense.stride(1) == 1
    rows, K = dense.shape
    if values is None:
        values = torch.empty((rows, K // 2), dtype=dense.dtype, device=dense.device)
    if meta is None:
        meta = torch.empty((rows, (K + 31) // 32), dtype=torch.int32, device=dense.device)
    st = lib().sp24_prune_compress(_code(dense), rows, K, _ptr(dense), dense.stride(0), _ptr(values),
                                   _ptr(meta), _stream(dense.device))
    _check("sp24_prune_compress", st)
    return values, meta


def quantize_prune_compress(x: torch.Tensor, values=None, meta=None, scales=None):
    """Per-row e4m3 quantization fused with the 2:4 prune and compress:
    (values rows x K/2 e4m3, meta rows x K/32 int32, scales rows fp32)."""
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, K = x.shape
    if values is None:
        values = torch.empty((rows, K // 2), dtype=torch.float8_e4m3fn, device=x.device)
    if meta is None:
        meta = torch.empty((rows, (K + 31) // 32), dtype=torch.int32, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    st = lib().sp24_quantize_prune_compress(_code(x), rows, K, _ptr(x), x.stride(0), _ptr(values), _ptr(meta),
                                            _ptr(scales), _stream(x.device))
    _check("sp24_quantize_prune_compress", st)
    return values, meta, scales


def quantize_e4m3(x: torch.Tensor, out=None, scales=None):
    """Per-row e4m3 quantization: (codes rows x K e4m3, scales rows fp32)."""
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, K = x.shape
    if out is None:
        out = torch.empty((rows, K), dtype=torch.float8_e4m3fn, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    st = lib().sp24_quantize_e4m3(_code(x), rows, K, _ptr(x), x.stride(0), _ptr(out), _ptr(scales),
                                  _stream(x.device))
    _check("sp24_quantize_e4m3", st)
    return out, scales


def decompress(values: torch.Tensor, meta: torch.Tensor, K: int, out=None):
    rows = values.shape[0]
    if out is None:
        out = torch.empty((rows, K), dtype=values.dtype, device=values.device)
    st = lib().sp24_decompress(_code(values), rows, K, _ptr(values), _ptr(meta), _ptr(out), out.stride(0),
                               _stream(values.device))
    _check("sp24_decompress", st)
    return out


def sp24_gemm(which: int, values, meta, dense, M: int, N: int, K: int, out_dtype=torch.bfloat16,
              scale_x=None, scale_w=None, out=None):
    """Y (M x N) = X W^T with W (which=SPARSE_W) or X (which=SPARSE_X) given as (values, meta)."""
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dense.device)
    st = lib().sp24_gemm(which, _code(dense), _code(out), M, N, K, _ptr(values), _ptr(meta), _ptr(dense),
                         _ptr(scale_x), _ptr(scale_w), _ptr(out), _stream(dense.device))
    _check("sp24_gemm", st)
    return out


def dense_gemm(x, w, out_dtype=torch.bfloat16, scale_x=None, scale_w=None, out=None):
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    st = lib().dense_gemm(_code(x), _code(out), M, N, K, _ptr(x), _ptr(w), _ptr(scale_x), _ptr(scale_w),
                          _ptr(out), _stream(x.device))
    _check("dense_gemm", st)
    return out


def hybrid_gemm(values, meta, w_dense, x, N_s: int, N_d: int, out_dtype=torch.bfloat16, scale_x=None,
                scale_w=None, out=None):
    """Y (M x (N_s + N_d)): columns [0, N_s) from the compressed rows (values, meta), the rest from the
    dense rows w_dense (N_d x K); one launch.  values / meta / w_dense may be None for an empty region."""
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N_s + N_d), dtype=out_dtype, device=x.device)
    st = lib().sp24_hybrid_gemm(_code(x), _code(out), M, N_s, N_d, K, _ptr(values), _ptr(meta), _ptr(w_dense),
                                _ptr(x), _ptr(scale_x), _ptr(scale_w), _ptr(out), _stream(x.device))
    _check("sp24_hybrid_gemm", st)
    return out


def hybrid_kernel(in_dtype, out_dtype, M: int, N_s: int, N_d: int, K: int):
    """Name of the kernel hybrid_gemm launches for this shape; None if rejected."""
    name = lib().sp24_hybrid_kernel(DTYPE_CODE[in_dtype], DTYPE_CODE[out_dtype], M, N_s, N_d, K)
    return None if name is None else name.decode()


def select_tactic(which, values, meta, dense_other, dense_pruned, M, N, K, out_dtype=torch.bfloat16,
                  scale_x=None, scale_w=None, y_scratch=None, warmup=5, reps=20):
    """Times sparse(+compress) against dense on these buffers; returns the tactic record."""
    dev = dense_other.device
    if y_scratch is None:
        y_scratch = torch.empty((M, N), dtype=out_dtype, device=dev)
    rec = Tactic()
    st = lib().sp24_select_tactic(which, _code(dense_other), _code(y_scratch), M, N, K, _ptr(values),
                                  _ptr(meta), _ptr(dense_other), _ptr(dense_pruned), _ptr(scale_x),
                                  _ptr(scale_w), _ptr(y_scratch), warmup, reps, _stream(dev),
                                  ctypes.byref(rec))
    _check("sp24_select_tactic", st)
    return rec.as_dict()


def tactic_decide(eligible: bool, t_sparse, t_dense) -> dict:
    """The decision rule alone on host timings (microseconds)."""
    ts = (ctypes.c_double * max(1, len(t_sparse)))(*t_sparse)
    td = (ctypes.c_double * max(1, len(t_dense)))(*t_dense)
    rec = Tactic()
    st = lib().sp24_tactic_decide(int(eligible), ts, len(t_sparse), td, len(t_dense), ctypes.byref(rec))
    _check("sp24_tactic_decide", st)
    return rec.as_dict()


def tactic_record(rec: dict) -> Tactic:
    """A record dict (as select_tactic returns) back in the C layout."""
    t = Tactic()
    t.eligible = int(bool(rec["eligible"]))
    t.selected = 1 if rec["selected"] == "sparse" else 0
    t.t_sparse_us, t.t_compress_us = float(rec["t_sparse_us"]), float(rec["t_compress_us"])
    t.t_dense_us, t.ratio = float(rec["t_dense_us"]), float(rec["ratio"])
    t.reason = rec["reason"].encode()[:95]
    t.kernel = rec["kernel"].encode()[:63]
    return t


def audit_aggregate(records, layer_counts, other_time_us: float = 0.0) -> dict:
    """Manifest metrics over per-shape tactic records (dicts), each shared by layer_counts[i] layers."""
    n = len(records)
    if len(layer_counts) != n:
        raise ValueError("one layer count per record")
    arr = (Tactic * max(1, n))(*[tactic_record(r) for r in records])
    cnt = (_i64 * max(1, n))(*[int(c) for c in layer_counts])
    out = AuditMetrics()
    _check("sp24_audit_aggregate", lib().sp24_audit_aggregate(arr, cnt, n, float(other_time_us),
                                                             ctypes.byref(out)))
    return out.as_dict()


def gemm_kernel(sparse: bool, which: int, in_dtype, out_dtype, M: int, N: int, K: int):
    """Name of the kernel sp24_gemm (sparse) or dense_gemm launches for this shape; None if rejected."""
    name = lib().sp24_gemm_kernel(int(sparse), which, DTYPE_CODE[in_dtype], DTYPE_CODE[out_dtype], M, N, K)
    return None if name is None else name.decode()


def version() -> str:
    return lib().sp24_version().decode()
