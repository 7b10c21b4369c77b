"""Helpers shared by the GPU tests: moving bit patterns between numpy and the
device, and the GEMM tolerance."""
import sys

import numpy as np
import torch

import oracle

TORCH_OF = {oracle.F16: torch.float16, oracle.BF16: torch.bfloat16, oracle.E4M3: torch.float8_e4m3fn,
            oracle.F32: torch.float32, oracle.I8: torch.int8}
VIEW_OF = {oracle.F16: torch.int16, oracle.BF16: torch.int16, oracle.E4M3: torch.uint8, oracle.F32: torch.int32,
           oracle.I8: torch.uint8}
NP_OF = {oracle.F16: np.uint16, oracle.BF16: np.uint16, oracle.E4M3: np.uint8, oracle.F32: np.uint32,
         oracle.I8: np.uint8}

# Parity bar for GEMM outputs: max |Y - R| / max(|R|, rms R).  fp16/bf16 inputs
# with fp32 accumulation: 1e-2; fp8 e4m3: 3e-2 (both sides on the same
# e4m3-decoded values); int8: 1e-2 (exact int32 sums, one conversion and
# the output rounding).  The error the arithmetic itself allows is far lower:
# one output rounding (bf16: 2^-9 relative) plus fp32 accumulation
# (~sqrt(K) * 2^-24 relative to sum |x w|).
TOL = {oracle.F16: 1e-2, oracle.BF16: 1e-2, oracle.E4M3: 3e-2, oracle.I8: 1e-2}


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, dt: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(NP_OF[dt]).view(
        {np.uint16: np.int16, np.uint8: np.uint8, np.uint32: np.int32}[NP_OF[dt]]))
    return t.view(VIEW_OF[dt]).view(TORCH_OF[dt]).cuda()


def to_host(t: torch.Tensor, dt: int) -> np.ndarray:
    return t.detach().contiguous().cpu().view(VIEW_OF[dt]).numpy().view(NP_OF[dt])


def meta_dev(m: np.ndarray) -> torch.Tensor:
    """Metadata words (uint32) as the int32 device tensor the binding takes."""
    return torch.from_numpy(np.ascontiguousarray(m, dtype=np.uint32).view(np.int32)).cuda()


def meta_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def decode_out(Y: torch.Tensor) -> np.ndarray:
    return Y.detach().float().cpu().numpy().astype(np.float64)


def band_rows(M: int, band: int = 256, seed: int = 0) -> np.ndarray:
    """Rows of M to compare at full size: all of them up to 64 rows; beyond,
    one row at a seeded place in every band of 256 rows (one per band of
    output tiles), plus rows 0 and M - 1."""
    if M <= 64:
        return np.arange(M, dtype=np.int64)
    rng = np.random.default_rng(seed + M)
    starts = np.arange(0, M, band)
    picks = starts + rng.integers(0, band, size=len(starts))
    return np.unique(np.clip(np.r_[0, picks, M - 1], 0, M - 1)).astype(np.int64)
