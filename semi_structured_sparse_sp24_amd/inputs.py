"""Seeded synthetic operands for 2:4 sparse GEMM workloads.

This module only draws random numbers and casts them to the storage formats;
it holds none of the sparse method's arithmetic (no pruning, packing or
multiplication).  Both the GPU path and the CPU oracle are fed the bytes it
returns, so the two sides always see identical inputs.

Everything is drawn on the host with ``torch.Generator('cpu')`` in fp32 and
cast with round-to-nearest-even.  Arrays come back as numpy bit patterns:
``uint16`` for fp16/bf16, ``uint8`` for fp8 e4m3 (OCP "e4m3fn").

Workloads, shaped like the linear layers of the pages' LLMs:
  tiny      W 256x256 fp16 ~N(0, 0.02), X 16x256 fp16 ~N(0, 1)
  decode    bf16 W (N, K) in {(4096,4096), (6144,4096), (28672,4096),
            (4096,14336)} ~N(0, 0.02); X of M in {1, 4, 16} rows ~N(0, 1)
  prefill   the same weights; M in {512, 2048, 8192}
  fp8       e4m3 W (N, K) in {(5120,5120), (51200,5120), (5120,25600)} with
            one fp32 scale per output channel, X e4m3 with one scale per token;
            M in {1, 64, 4096}; bf16 output
  online    X 4096x4096 bf16 ~N(0, 1) with 1% of entries scaled x20, the
            activation being the operand that is pruned on every call;
            W 4096x4096 bf16 ~N(0, 0.02)
  online_fp8  the same X (bf16, outliers), quantized to e4m3 per row and
            pruned on every call by the library; W e4m3 (N, K) in
            {(4096,4096), (28672,4096)} with per-channel scales; M = 4096
  online_int8  the same X, quantized to symmetric int8 per row and pruned on
            every call by the library; W int8 (N, K) in {(4096,4096),
            (28672,4096)} with per-channel scales; M = 4096
  int8      the fp8 shapes in symmetric per-row int8
  hybrid    the prefill weights, the last N/8 rows kept dense; M in {2048, 8192}
  ksplit    the prefill weights, the last K/4 columns kept dense; M in {2048, 8192}
Seed of tensor t (0 = W, 1 = X, 2 = outlier mask) of shape s in workload c at
M index j:  10000*c + 100*s + 10*t + j.
"""
from __future__ import annotations

import numpy as np
import torch

F16, BF16, E4M3, F32, I8 = 0, 1, 2, 3, 4
FP8_MAX = 448.0
I8_MAX = 127.0

TORCH_DTYPE = {F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.float8_e4m3fn,
               F32: torch.float32, I8: torch.int8}
BITS_DTYPE = {F16: np.uint16, BF16: np.uint16, E4M3: np.uint8, F32: np.uint32, I8: np.uint8}
ELEM_BYTES = {F16: 2, BF16: 2, E4M3: 1, F32: 4, I8: 1}

WORKLOADS = {
    "tiny": dict(index=1, dtype=F16, out=F16, shapes=[(256, 256)], ms=[16]),
    "decode": dict(index=2, dtype=BF16, out=BF16,
                   shapes=[(4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336)],
                   ms=[1, 4, 16]),
    "prefill": dict(index=3, dtype=BF16, out=BF16,
                    shapes=[(4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336)],
                    ms=[512, 2048, 8192]),
    "fp8": dict(index=4, dtype=E4M3, out=BF16,
                shapes=[(5120, 5120), (51200, 5120), (5120, 25600)], ms=[1, 64, 4096]),
    "online": dict(index=5, dtype=BF16, out=BF16, shapes=[(4096, 4096)], ms=[4096]),
    "online_fp8": dict(index=6, dtype=E4M3, act=BF16, out=BF16, shapes=[(4096, 4096), (28672, 4096)],
                       ms=[4096]),
    "online_int8": dict(index=10, dtype=I8, act=BF16, out=BF16, shapes=[(4096, 4096), (28672, 4096)],
                        ms=[4096]),
    # the fp8 shapes in symmetric per-row int8 (the 2:4 + INT8 variant)
    "int8": dict(index=8, dtype=I8, out=BF16,
                 shapes=[(5120, 5120), (51200, 5120), (5120, 25600)], ms=[1, 64, 4096]),
    # the prefill layers with one output row in eight kept dense (hybrid_split)
    "hybrid": dict(index=7, dtype=BF16, out=BF16,
                   shapes=[(4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336)], ms=[2048, 8192]),
    # the prefill layers with the last quarter of K kept dense (ksplit_split)
    "ksplit": dict(index=9, dtype=BF16, out=BF16,
                   shapes=[(4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336)], ms=[2048, 8192]),
}


def hybrid_split(N: int) -> tuple[int, int]:
    """(sparse rows, dense rows) of an N-row weight in the hybrid workload: the
    last N/8 rows (a multiple of 256) stay dense."""
    nd = max(256, N // 8 // 256 * 256)
    return N - nd, nd


def ksplit_split(K: int) -> tuple[int, int]:
    """(2:4 columns, dense columns) of a K-wide weight in the ksplit workload:
    the last K/4 columns (a multiple of 256) stay dense."""
    kd = max(256, K // 4 // 256 * 256)
    return K - kd, kd


def seed_of(c: int, s: int, t: int, j: int) -> int:
    return 10000 * c + 100 * s + 10 * t + j


def normal(shape, sigma: float, seed: int) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32) * sigma


def to_bits(t: torch.Tensor, dt: int) -> np.ndarray:
    """Cast an fp32 tensor to format dt (RNE) and return its bit patterns."""
    q = t.to(TORCH_DTYPE[dt]).contiguous()
    view = {F16: torch.int16, BF16: torch.int16, E4M3: torch.uint8, F32: torch.int32}[dt]
    return q.view(view).numpy().view(BITS_DTYPE[dt]).copy()


def quantize_e4m3_rows(t: torch.Tensor):
    """One fp32 scale per row (absmax / 448; 1 for an all-zero row), values
    clamped to +-448 and cast to e4m3fn with RNE.  Returns (bits, scales)."""
    absmax = t.abs().amax(dim=1)
    scale = torch.where(absmax > 0, absmax / FP8_MAX, torch.ones_like(absmax)).to(torch.float32)
    q = (t / scale[:, None]).clamp(-FP8_MAX, FP8_MAX)
    return to_bits(q, E4M3), scale.numpy().astype(np.float32)


def quantize_i8_rows(t: torch.Tensor):
    """Symmetric int8 with one fp32 scale per row (absmax / 127; 1 for an
    all-zero row): round half to even, clamp to +-127.  Returns (bits as
    uint8, scales)."""
    absmax = t.abs().amax(dim=1)
    scale = torch.where(absmax > 0, absmax / I8_MAX, torch.ones_like(absmax)).to(torch.float32)
    q = torch.round(t / scale[:, None]).clamp(-I8_MAX, I8_MAX).to(torch.int8)
    return q.numpy().view(np.uint8).copy(), scale.numpy().astype(np.float32)


def outliers(t: torch.Tensor, frac: float, factor: float, seed: int) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(int(seed))
    mask = torch.rand(*t.shape, generator=g) < frac
    return torch.where(mask, t * factor, t)


def weight(workload: str, s: int):
    """(bits, scale or None) of weight shape index s of a workload."""
    w = WORKLOADS[workload]
    N, K = w["shapes"][s]
    t = normal((N, K), 0.02, seed_of(w["index"], s, 0, 0))
    if w["dtype"] == E4M3:
        return quantize_e4m3_rows(t)
    if w["dtype"] == I8:
        return quantize_i8_rows(t)
    return to_bits(t, w["dtype"]), None


def activation(workload: str, s: int, j: int, M: int | None = None):
    """(bits, scale or None) of the X operand for weight shape s and M index j."""
    w = WORKLOADS[workload]
    N, K = w["shapes"][s]
    if M is None:
        M = w["ms"][j]
    t = normal((M, K), 1.0, seed_of(w["index"], s, 1, j))
    if workload in ("online", "online_fp8", "online_int8"):
        t = outliers(t, 0.01, 20.0, seed_of(w["index"], s, 2, j))
    act = w.get("act", w["dtype"])
    if act == E4M3:
        return quantize_e4m3_rows(t)
    if act == I8:
        return quantize_i8_rows(t)
    return to_bits(t, act), None


def integer_operand(shape, seed: int, dt: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Entries drawn uniformly from the integers lo..hi (exact in every format)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    t = torch.randint(lo, hi + 1, tuple(shape), generator=g).to(torch.float32)
    return to_bits(t, dt)


def uniform_bits(shape, seed: int, dt: int) -> np.ndarray:
    """Uniformly random bit patterns of format dt (every value class, NaN and
    Inf included)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    hi = 256 if dt == E4M3 else 65536
    t = torch.randint(0, hi, tuple(shape), generator=g, dtype=torch.int64)
    return t.numpy().astype(BITS_DTYPE[dt])
