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
  quantize_i8_prune_compress(x) -> (values int8, meta, scales): fused online int8 path
  quantize_i8(x)               -> (codes int8, scales): its dense side
  hybrid_gemm(...)             -> Y = X [Ws | Wd]^T, Ws compressed and Wd dense rows, one launch
  ksplit_gemm(...)             -> Y = X W^T, W's first K_s columns compressed and the rest dense, one launch
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
    "sp24_ksplit_gemm": (_i32, [_i32, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sp24_ksplit_kernel": (ctypes.c_char_p, [_i32, _i32, _i64, _i64, _i64, _i64]),
    "sp24_audit_aggregate": (_i32, [ctypes.POINTER(Tactic), ctypes.POINTER(_i64), _i64, _dbl,
                                    ctypes.POINTER(AuditMetrics)]),
    "sp24_quantize_prune_compress": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp]),
    "sp24_quantize_e4m3": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "sp24_quantize_i8_prune_compress": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp]),
    "sp24_quantize_i8": (_i32, [_i32, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
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


# ---------------------------------------------------------------- argument checks
# The kernels size their buffer descriptors and grids from M, N and K alone, so
# every tensor is checked against them here, before anything reaches the
# library: shape, row stride, contiguity of K, dtype, and one common device.
# Shape, stride and dtype mismatches raise ValueError / TypeError; a tensor
# not on a GPU, or on another GPU than the rest, raises ValueError.

def _mat(t, name, rows, cols, dtype=None, ld_min=None):
    """t is a rows x cols matrix with contiguous columns.  Its row stride must
    equal cols, or (ld_min given) be at least ld_min."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != 2 or tuple(t.shape) != (int(rows), int(cols)):
        raise ValueError(f"{name} must have shape ({rows}, {cols}), got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if rows > 0 and cols > 0:
        if cols > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must be contiguous along its last axis (stride(1) == 1)")
        if rows > 1:
            if ld_min is None and t.stride(0) != cols:
                raise ValueError(f"{name} must be row-major contiguous (stride(0) == {cols}), "
                                 f"got stride {t.stride()}")
            if ld_min is not None and t.stride(0) < ld_min:
                raise ValueError(f"{name} row stride {t.stride(0)} is below {ld_min}")
    return t


def _vec(t, name, n):
    """An optional fp32 vector of n contiguous elements (None passes)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if t.dim() != 1 or t.shape[0] != int(n):
        raise ValueError(f"{name} must have shape ({n},), got {tuple(t.shape)}")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be torch.float32, got {t.dtype}")
    if n > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(*ts):
    """Every tensor given (None skipped) sits on one GPU; returns that device."""
    ts = [t for t in ts if t is not None]
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError(f"every operand must be on a GPU, found one on {t.device}")
        if t.device != dev:
            raise ValueError(f"operands on different devices: {dev} and {t.device}")
    return dev


def _compressed(values, meta, rows, K, dtype, what):
    """(values, meta) of a rows x K operand in the library's compressed form."""
    _mat(values, f"{what} values", rows, K // 2, dtype)
    _mat(meta, f"{what} meta", rows, (K + 31) // 32, torch.int32)


def meta_words_per_row(K: int) -> int:
    return int(lib().sp24_meta_words_per_row(K))


def prune_compress(dense: torch.Tensor, values=None, meta=None):
    """Magnitude 2:4 along the last axis: (values rows x K/2, meta rows x ceil(K/32) int32)."""
    if not isinstance(dense, torch.Tensor) or dense.dim() != 2:
        raise ValueError("prune_compress takes a 2-D tensor")
    rows, K = dense.shape
    _mat(dense, "dense", rows, K, ld_min=K)
    if values is None:
        values = torch.empty((rows, K // 2), dtype=dense.dtype, device=dense.device)
    if meta is None:
        meta = torch.empty((rows, (K + 31) // 32), dtype=torch.int32, device=dense.device)
    _compressed(values, meta, rows, K, dense.dtype, "output")
    _same_device(dense, values, meta)
    ld = dense.stride(0) if rows > 1 else K
    st = lib().sp24_prune_compress(_code(dense), rows, K, _ptr(dense), ld, _ptr(values),
                                   _ptr(meta), _stream(dense.device))
    _check("sp24_prune_compress", st)
    return values, meta


def _quantize_pruned(fn, code_dtype, x, values, meta, scales):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{fn} takes a 2-D tensor")
    rows, K = x.shape
    _mat(x, "x", rows, K, ld_min=K)
    if values is None:
        values = torch.empty((rows, K // 2), dtype=code_dtype, device=x.device)
    if meta is None:
        meta = torch.empty((rows, (K + 31) // 32), dtype=torch.int32, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _compressed(values, meta, rows, K, code_dtype, "output")
    _vec(scales, "scales", rows)
    _same_device(x, values, meta, scales)
    ld = x.stride(0) if rows > 1 else K
    st = getattr(lib(), "sp24_" + fn)(_code(x), rows, K, _ptr(x), ld, _ptr(values), _ptr(meta), _ptr(scales),
                                      _stream(x.device))
    _check("sp24_" + fn, st)
    return values, meta, scales


def _quantize_codes(fn, code_dtype, x, out, scales):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{fn} takes a 2-D tensor")
    rows, K = x.shape
    _mat(x, "x", rows, K, ld_min=K)
    if out is None:
        out = torch.empty((rows, K), dtype=code_dtype, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _mat(out, "out", rows, K, code_dtype)
    _vec(scales, "scales", rows)
    _same_device(x, out, scales)
    ld = x.stride(0) if rows > 1 else K
    st = getattr(lib(), "sp24_" + fn)(_code(x), rows, K, _ptr(x), ld, _ptr(out), _ptr(scales), _stream(x.device))
    _check("sp24_" + fn, st)
    return out, scales


def quantize_prune_compress(x: torch.Tensor, values=None, meta=None, scales=None):
    """Per-row e4m3 quantization fused with the 2:4 prune and compress:
    (values rows x K/2 e4m3, meta rows x K/32 int32, scales rows fp32)."""
    return _quantize_pruned("quantize_prune_compress", torch.float8_e4m3fn, x, values, meta, scales)


def quantize_e4m3(x: torch.Tensor, out=None, scales=None):
    """Per-row e4m3 quantization: (codes rows x K e4m3, scales rows fp32)."""
    return _quantize_codes("quantize_e4m3", torch.float8_e4m3fn, x, out, scales)


def quantize_i8_prune_compress(x: torch.Tensor, values=None, meta=None, scales=None):
    """Per-row symmetric int8 quantization fused with the 2:4 prune and
    compress: (values rows x K/2 int8, meta rows x K/32 int32, scales rows fp32)."""
    return _quantize_pruned("quantize_i8_prune_compress", torch.int8, x, values, meta, scales)


def quantize_i8(x: torch.Tensor, out=None, scales=None):
    """Per-row symmetric int8 quantization: (codes rows x K int8, scales rows fp32)."""
    return _quantize_codes("quantize_i8", torch.int8, x, out, scales)


def decompress(values: torch.Tensor, meta: torch.Tensor, K: int, out=None):
    """The dense rows x K operand: kept values in place, +0 elsewhere."""
    if not isinstance(values, torch.Tensor) or values.dim() != 2:
        raise ValueError("decompress takes 2-D values")
    rows = values.shape[0]
    _compressed(values, meta, rows, K, values.dtype, "input")
    if out is None:
        out = torch.empty((rows, K), dtype=values.dtype, device=values.device)
    _mat(out, "out", rows, K, values.dtype, ld_min=K)
    _same_device(values, meta, out)
    ld = out.stride(0) if rows > 1 else K
    st = lib().sp24_decompress(_code(values), rows, K, _ptr(values), _ptr(meta), _ptr(out), ld,
                               _stream(values.device))
    _check("sp24_decompress", st)
    return out


def _out(out, M, N, out_dtype, device):
    if out is None:
        return torch.empty((M, N), dtype=out_dtype, device=device)
    return _mat(out, "out", M, N)


def sp24_gemm(which: int, values, meta, dense, M: int, N: int, K: int, out_dtype=torch.bfloat16,
              scale_x=None, scale_w=None, out=None):
    """Y (M x N) = X W^T with W (which=SPARSE_W) or X (which=SPARSE_X) given as (values, meta)."""
    if which not in (SPARSE_W, SPARSE_X):
        raise ValueError(f"which must be SPARSE_W or SPARSE_X, got {which}")
    if not isinstance(dense, torch.Tensor):
        raise TypeError("dense must be a torch.Tensor")
    rows, other = (N, M) if which == SPARSE_W else (M, N)
    _mat(dense, "dense", other, K)
    _compressed(values, meta, rows, K, dense.dtype, "compressed operand")
    _vec(scale_x, "scale_x", M)
    _vec(scale_w, "scale_w", N)
    out = _out(out, M, N, out_dtype, dense.device)
    _same_device(dense, values, meta, scale_x, scale_w, out)
    st = lib().sp24_gemm(which, _code(dense), _code(out), M, N, K, _ptr(values), _ptr(meta), _ptr(dense),
                         _ptr(scale_x), _ptr(scale_w), _ptr(out), _stream(dense.device))
    _check("sp24_gemm", st)
    return out


def dense_gemm(x, w, out_dtype=torch.bfloat16, scale_x=None, scale_w=None, out=None):
    """Y (M x N) = X W^T on dense operands, the baseline and the fallback."""
    if not isinstance(x, torch.Tensor) or not isinstance(w, torch.Tensor) or x.dim() != 2 or w.dim() != 2:
        raise ValueError("dense_gemm takes 2-D tensors")
    M, K = x.shape
    N = w.shape[0]
    _mat(x, "x", M, K)
    _mat(w, "w", N, K, x.dtype)
    _vec(scale_x, "scale_x", M)
    _vec(scale_w, "scale_w", N)
    out = _out(out, M, N, out_dtype, x.device)
    _same_device(x, w, scale_x, scale_w, out)
    st = lib().dense_gemm(_code(x), _code(out), M, N, K, _ptr(x), _ptr(w), _ptr(scale_x), _ptr(scale_w),
                          _ptr(out), _stream(x.device))
    _check("dense_gemm", st)
    return out


def hybrid_gemm(values, meta, w_dense, x, N_s: int, N_d: int, out_dtype=torch.bfloat16, scale_x=None,
                scale_w=None, out=None):
    """Y (M x (N_s + N_d)): columns [0, N_s) from the compressed rows (values, meta), the rest from the
    dense rows w_dense (N_d x K); one launch.  values / meta / w_dense may be None for an empty region."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("hybrid_gemm takes a 2-D x")
    M, K = x.shape
    _mat(x, "x", M, K)
    if N_s > 0 or values is not None or meta is not None:
        _compressed(values, meta, N_s, K, x.dtype, "sparse rows")
    if N_d > 0 or w_dense is not None:
        _mat(w_dense, "w_dense", N_d, K, x.dtype)
    _vec(scale_x, "scale_x", M)
    _vec(scale_w, "scale_w", N_s + N_d)
    out = _out(out, M, N_s + N_d, out_dtype, x.device)
    _same_device(x, values, meta, w_dense, scale_x, scale_w, out)
    st = lib().sp24_hybrid_gemm(_code(x), _code(out), M, N_s, N_d, K, _ptr(values), _ptr(meta), _ptr(w_dense),
                                _ptr(x), _ptr(scale_x), _ptr(scale_w), _ptr(out), _stream(x.device))
    _check("sp24_hybrid_gemm", st)
    return out


def hybrid_kernel(in_dtype, out_dtype, M: int, N_s: int, N_d: int, K: int):
    """Name of the kernel hybrid_gemm launches for this shape; None if rejected."""
    name = lib().sp24_hybrid_kernel(DTYPE_CODE[in_dtype], DTYPE_CODE[out_dtype], M, N_s, N_d, K)
    return None if name is None else name.decode()


def ksplit_gemm(values, meta, w_dense, x, N: int, K_s: int, out_dtype=torch.bfloat16, scale_x=None,
                scale_w=None, out=None):
    """Y (M x N) = X W^T with W's columns [0, K_s) given compressed (values N x K_s/2, meta) and
    columns [K_s, K) dense (w_dense N x (K - K_s)); one launch.  values / meta may be None when
    K_s == 0, w_dense when K_s == K."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("ksplit_gemm takes a 2-D x")
    M, K = x.shape
    if not 0 <= K_s <= K:
        raise ValueError(f"K_s must lie in [0, {K}], got {K_s}")
    _mat(x, "x", M, K)
    if K_s > 0 or values is not None or meta is not None:
        _compressed(values, meta, N, K_s, x.dtype, "2:4 range")
    if K_s < K or w_dense is not None:
        _mat(w_dense, "w_dense", N, K - K_s, x.dtype)
    _vec(scale_x, "scale_x", M)
    _vec(scale_w, "scale_w", N)
    out = _out(out, M, N, out_dtype, x.device)
    _same_device(x, values, meta, w_dense, scale_x, scale_w, out)
    st = lib().sp24_ksplit_gemm(_code(x), _code(out), M, N, K_s, K, _ptr(values), _ptr(meta), _ptr(w_dense),
                                _ptr(x), _ptr(scale_x), _ptr(scale_w), _ptr(out), _stream(x.device))
    _check("sp24_ksplit_gemm", st)
    return out


def ksplit_kernel(in_dtype, out_dtype, M: int, N: int, K_s: int, K: int):
    """Name of the kernel ksplit_gemm launches for this shape; None if rejected."""
    name = lib().sp24_ksplit_kernel(DTYPE_CODE[in_dtype], DTYPE_CODE[out_dtype], M, N, K_s, K)
    return None if name is None else name.decode()


def select_tactic(which, values, meta, dense_other, dense_pruned, M, N, K, out_dtype=torch.bfloat16,
                  scale_x=None, scale_w=None, y_scratch=None, warmup=5, reps=20):
    """Times sparse(+compress) against dense on these buffers; returns the tactic record."""
    if which not in (SPARSE_W, SPARSE_X):
        raise ValueError(f"which must be SPARSE_W or SPARSE_X, got {which}")
    if not isinstance(dense_other, torch.Tensor):
        raise TypeError("dense_other must be a torch.Tensor")
    rows, other = (N, M) if which == SPARSE_W else (M, N)
    _mat(dense_other, "dense_other", other, K)
    _mat(dense_pruned, "dense_pruned", rows, K, dense_other.dtype)
    _compressed(values, meta, rows, K, dense_other.dtype, "compressed operand")
    _vec(scale_x, "scale_x", M)
    _vec(scale_w, "scale_w", N)
    dev = dense_other.device
    y_scratch = _out(y_scratch, M, N, out_dtype, dev)
    _same_device(dense_other, dense_pruned, values, meta, scale_x, scale_w, y_scratch)
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
