"""Benchmark of the 2:4 sparse GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

A step is one pass of the whole hot path over the workload's synthetic,
seeded operands: for every weight shape, prune+compress the weight (or, for
the online workload, the activation), decompress it (the dense pruned weight
the fallback uses), then for every M the sparse GEMM and the dense GEMM on
the same shapes.  Every kernel is timed with HIP events on the stream it runs
on; HBM-bound kernels run "cold" (an untimed read of a 1 GiB buffer before
each evicts L2 and the 256 MB Infinity Cache), compute-bound ones "warm".
After the timed steps the per-shape tactic (sparse iff faster) is selected
and the CPU oracle is timed on the host cores.  Rank 0 prints one JSON line.

Workloads (default: decode, the bf16 Llama-3-8B-like decode layers):
  tiny | decode | prefill | fp8 | online
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import semi_structured_sparse_sp24_amd as sp  # noqa: E402
from semi_structured_sparse_sp24_amd import inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
SPARSE_PEAK_TFLOPS = {inputs.BF16: 5033.0, inputs.F16: 5033.0, inputs.E4M3: 10066.0}   # 2:4, dense-equivalent
DENSE_PEAK_TFLOPS = {inputs.BF16: 2516.0, inputs.F16: 2516.0, inputs.E4M3: 5033.0}
DTYPE_NAME = {inputs.F16: "f16", inputs.BF16: "bf16", inputs.E4M3: "e4m3"}
TORCH = {inputs.F16: torch.float16, inputs.BF16: torch.bfloat16, inputs.E4M3: torch.float8_e4m3fn}


def dev(bits, dt):
    view = {np.uint16: np.int16, np.uint8: np.uint8}[bits.dtype.type]
    return torch.from_numpy(bits.view(view)).view(TORCH[dt]).cuda()


# ---------------------------------------------------------------- algorithmic bytes / flops

def sparse_gemm_bytes(M, N, K, eb, out_eb, sparse_rows, scales):
    """Compressed operand (values + meta) + dense operand + output (+ scales)."""
    other = N if sparse_rows == M else M
    return sparse_rows * K * eb // 2 + sparse_rows * K // 8 + other * K * eb + M * N * out_eb + \
        (4 * (M + N) if scales else 0)


def dense_gemm_bytes(M, N, K, eb, out_eb, scales):
    return (M + N) * K * eb + M * N * out_eb + (4 * (M + N) if scales else 0)


def compress_bytes(R, K, eb):
    return R * K * eb + R * K * eb // 2 + R * K // 8


def traffic_per_launch(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload`, from the FETCH_SIZE and WRITE_SIZE counter runs
    recorded in profiles/traffic.md (scaled by the same counters' reading for a copy of known size).
    None when no record exists or when the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        # | kernel | workload | source sha256 (12) | bytes per launch | ...
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) < 4 or cells[0] != kernel or cells[1] != workload:
            continue
        src = os.path.join(ROOT, "semi_structured_sparse_sp24_amd", "csrc", cells[2].split(":")[0])
        if not os.path.exists(src):
            return None
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:12]
        if cells[2].split(":")[1] != digest:
            return None
        return float(cells[3])
    return None


class Timer:
    """HIP events on torch's current stream (the one the library launches on)."""

    def __init__(self):
        self.pending = []           # (key, start, end)

    def time(self, key, fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pending.append((key, a, b))

    def collect(self):
        torch.cuda.synchronize()
        out = {}
        for key, a, b in self.pending:
            out.setdefault(key, []).append(a.elapsed_time(b) * 1e3)   # microseconds
        self.pending = []
        return out


def build_cases(workload):
    w = inputs.WORKLOADS[workload]
    dt, out = w["dtype"], w["out"]
    cases = []
    for s, (N, K) in enumerate(w["shapes"]):
        wb, sw = inputs.weight(workload, s)
        W = dev(wb, dt)
        shape = {"s": s, "N": N, "K": K, "W": W,
                 "sw": None if sw is None else torch.from_numpy(sw).cuda(), "ms": []}
        v, m = sp.prune_compress(W)
        shape["v"], shape["m"] = v, m
        shape["Wp"] = sp.decompress(v, m, K)
        for j, M in enumerate(w["ms"]):
            xb, sx = inputs.activation(workload, s, j)
            X = dev(xb, dt)
            item = {"j": j, "M": M, "X": X, "sx": None if sx is None else torch.from_numpy(sx).cuda(),
                    "Y": torch.empty((M, N), dtype=TORCH[out] if out in TORCH else torch.float32, device="cuda"),
                    "Yd": torch.empty((M, N), dtype=TORCH[out] if out in TORCH else torch.float32, device="cuda")}
            if workload == "online":
                item["xv"] = torch.empty((M, K // 2), dtype=TORCH[dt], device="cuda")
                item["xm"] = torch.empty((M, (K + 31) // 32), dtype=torch.int32, device="cuda")
            shape["ms"].append(item)
        cases.append(shape)
    torch.cuda.synchronize()
    return cases


def run_step(workload, cases, timer, flush, cold):
    w = inputs.WORKLOADS[workload]
    dt = w["dtype"]
    for c in cases:
        N, K = c["N"], c["K"]
        if workload != "online":
            if cold:
                flush.sum()
            timer.time(("compress", c["s"]), lambda: sp.prune_compress(c["W"], values=c["v"], meta=c["m"]))
            if cold:
                flush.sum()
            timer.time(("decompress", c["s"]), lambda: sp.decompress(c["v"], c["m"], K, out=c["Wp"]))
        for it in c["ms"]:
            M = it["M"]
            if workload == "online":
                # the activation is the sparse operand: prune+compress it on every call
                timer.time(("compress", c["s"], it["j"]),
                           lambda: sp.prune_compress(it["X"], values=it["xv"], meta=it["xm"]))
                timer.time(("sparse", c["s"], it["j"]),
                           lambda: sp.sp24_gemm(sp.SPARSE_X, it["xv"], it["xm"], c["W"], M, N, K, out=it["Y"]))
                timer.time(("dense", c["s"], it["j"]), lambda: sp.dense_gemm(it["X"], c["W"], out=it["Yd"]))
                continue
            if cold:
                flush.sum()
            timer.time(("sparse", c["s"], it["j"]),
                       lambda: sp.sp24_gemm(sp.SPARSE_W, c["v"], c["m"], it["X"], M, N, K,
                                            scale_x=it["sx"], scale_w=c["sw"], out=it["Y"]))
            if cold:
                flush.sum()
            timer.time(("dense", c["s"], it["j"]),
                       lambda: sp.dense_gemm(it["X"], c["Wp"], scale_x=it["sx"], scale_w=c["sw"], out=it["Yd"]))


def cpu_baseline(workload, budget_s):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: its GEMMs (fp64 on the decompressed weight) for as many
    (shape, M) cases as fit the time budget, rows of M sampled when M is large."""
    import oracle

    w = inputs.WORKLOADS[workload]
    dt = w["dtype"]
    flops = 0.0
    secs = 0.0
    done = []
    t_start = time.perf_counter()
    for s, (N, K) in enumerate(w["shapes"]):
        if secs > budget_s or time.perf_counter() - t_start > 3 * budget_s:
            break
        wb, sw = inputs.weight(workload, s)
        if workload != "online":
            wv, wm = oracle.prune_compress(dt, wb)
        for j, M in enumerate(w["ms"]):
            if secs > budget_s or time.perf_counter() - t_start > 3 * budget_s:
                break
            xb, sx = inputs.activation(workload, s, j)
            rows = M if M <= 64 else 16
            mrows = np.linspace(0, M - 1, rows).astype(np.int64)
            if workload == "online":
                xv, xm = oracle.prune_compress(dt, xb)
                t0 = time.perf_counter()
                oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, mrows=mrows)
            else:
                t0 = time.perf_counter()
                oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw, mrows=mrows)
            secs += time.perf_counter() - t0
            flops += 2.0 * rows * N * K
            done.append(f"({N},{K})xM{M}" + ("" if rows == M else f"[{rows} rows]"))
    return {"value": flops / secs / 1e12 if secs > 0 else None, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"oracle fp64 GEMM on the decompressed operand, {len(done)} cases: " + " ".join(done) +
                      f"; {secs:.1f} s of GEMM time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=list(inputs.WORKLOADS))
    ap.add_argument("--cold", choices=["auto", "on", "off"], default="auto")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle GEMM time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tactic", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path runs on a single MI355X; multi-GPU sharding is a "
              "design note only (see the design notes), so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sp.lib()                                   # fails loudly if the HIP library is missing

    workload = args.workload
    w = inputs.WORKLOADS[workload]
    dt, out = w["dtype"], w["out"]
    eb, out_eb = inputs.ELEM_BYTES[dt], inputs.ELEM_BYTES[out]
    cold = (workload in ("decode", "fp8", "tiny")) if args.cold == "auto" else args.cold == "on"
    scales = dt == inputs.E4M3

    cases = build_cases(workload)
    # cold runs read (not write) a 1 GiB buffer before each timed kernel: that evicts L2 and the
    # 256 MB Infinity Cache without leaving dirty lines whose write-back would compete with the kernel
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda") if cold else None
    timer = Timer()
    for _ in range(args.warmup):
        run_step(workload, cases, timer, flush, cold)
    timer.collect()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(workload, cases, timer, flush, cold)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = timer.collect()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        b.copy_(a)
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- per-case table
    med = lambda k: float(np.median(times[k]))
    rows = []
    tot = {"sparse_t": 0.0, "dense_t": 0.0, "flops": 0.0, "sparse_bytes": 0.0, "compress_t": 0.0,
           "compress_bytes": 0.0, "sparse_launches": 0}
    for c in cases:
        N, K = c["N"], c["K"]
        for it in c["ms"]:
            M = it["M"]
            key = (c["s"], it["j"])
            ts = times[("sparse",) + key]
            td = times[("dense",) + key]
            sparse_rows = M if workload == "online" else N
            sb = sparse_gemm_bytes(M, N, K, eb, out_eb, sparse_rows, scales)
            db = dense_gemm_bytes(M, N, K, eb, out_eb, scales)
            fl = 2.0 * M * N * K
            tsm, tdm = float(np.median(ts)), float(np.median(td))
            row = {"N": N, "K": K, "M": M, "t_sparse_us": round(tsm, 2), "t_dense_us": round(tdm, 2),
                   "speedup": round(tdm / tsm, 3),
                   "sparse_tflops": round(fl / tsm / 1e6, 1), "dense_tflops": round(fl / tdm / 1e6, 1),
                   "sparse_GBps": round(sb / tsm / 1e3, 1), "dense_GBps": round(db / tdm / 1e3, 1),
                   "sparse_hbm_frac": round(sb / tsm / 1e3 / HBM_PEAK_GBPS, 3),
                   "sparse_mfma_frac": round(fl / tsm / 1e6 / SPARSE_PEAK_TFLOPS[dt], 3)}
            if workload == "online":
                tc = float(np.median(times[("compress",) + key]))
                row["t_compress_us"] = round(tc, 2)
                row["speedup_incl_compress"] = round(tdm / (tc + tsm), 3)
                tot["compress_t"] += sum(times[("compress",) + key])
                tot["compress_bytes"] += compress_bytes(M, K, eb) * len(times[("compress",) + key])
            rows.append(row)
            tot["sparse_t"] += sum(ts)
            tot["dense_t"] += sum(td)
            tot["flops"] += fl * len(ts)
            tot["sparse_bytes"] += sb * len(ts)
            tot["sparse_launches"] += len(ts)
        if workload != "online":
            tcs = times[("compress", c["s"])]
            tot["compress_t"] += sum(tcs)
            tot["compress_bytes"] += compress_bytes(N, K, eb) * len(tcs)

    value = tot["flops"] / tot["sparse_t"] / 1e6                    # TFLOP/s (dense-equivalent)
    speedup = tot["dense_t"] / tot["sparse_t"]
    compress_gbps = tot["compress_bytes"] / tot["compress_t"] / 1e3

    # roofline of the dominant kernel: the sparse GEMM kernel (by name, as the dispatch picks it per
    # shape) with the largest share of the step's sparse GEMM time; achieved = its algorithmic bytes
    # (HBM-bound decode) or flops (MFMA-bound prefill) per launch / its mean launch duration
    per_kernel = {}
    for c in cases:
        for it in c["ms"]:
            M, N, K = it["M"], c["N"], c["K"]
            which = sp.SPARSE_X if workload == "online" else sp.SPARSE_W
            name = sp.gemm_kernel(True, which, TORCH[dt], it["Y"].dtype, M, N, K)
            ts = times[("sparse", c["s"], it["j"])]
            sparse_rows = M if workload == "online" else N
            k = per_kernel.setdefault(name, {"t": 0.0, "n": 0, "bytes": 0.0, "flops": 0.0})
            k["t"] += sum(ts)
            k["n"] += len(ts)
            k["bytes"] += sparse_gemm_bytes(M, N, K, eb, out_eb, sparse_rows, scales) * len(ts)
            k["flops"] += 2.0 * M * N * K * len(ts)
    kname = max(per_kernel, key=lambda n: per_kernel[n]["t"])
    k = per_kernel[kname]
    avg_us = k["t"] / k["n"]
    hbm_bound = max(it["M"] for c in cases for it in c["ms"]) <= 64
    if hbm_bound:
        achieved = k["bytes"] / k["t"] / 1e3
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_per_launch(kname, workload),
                "kernel": kname, "launches": k["n"], "bytes_per_launch": round(k["bytes"] / k["n"]),
                "avg_launch_us": round(avg_us, 3)}
    else:
        peak = SPARSE_PEAK_TFLOPS[dt]
        achieved = k["flops"] / k["t"] / 1e6
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_per_launch(kname, workload),
                "kernel": kname, "launches": k["n"], "flops_per_launch": round(k["flops"] / k["n"]),
                "avg_launch_us": round(avg_us, 3)}
    roof["kernels"] = {n: {"launches": v["n"], "avg_launch_us": round(v["t"] / v["n"], 3),
                           "share": round(v["t"] / tot["sparse_t"], 3)} for n, v in per_kernel.items()}

    tactics = []
    if not args.no_tactic:
        for c in cases:
            for it in c["ms"]:
                M, N, K = it["M"], c["N"], c["K"]
                if workload == "online":
                    rec = sp.select_tactic(sp.SPARSE_X, it["xv"], it["xm"], c["W"], it["X"], M, N, K,
                                           y_scratch=it["Y"], warmup=3, reps=10)
                else:
                    rec = sp.select_tactic(sp.SPARSE_W, c["v"], c["m"], it["X"], c["Wp"], M, N, K,
                                           scale_x=it["sx"], scale_w=c["sw"], y_scratch=it["Y"], warmup=3,
                                           reps=10)
                tactics.append({"N": N, "K": K, "M": M, "selected": rec["selected"], "ratio": round(rec["ratio"], 3),
                                "reason": rec["reason"], "kernel": rec["kernel"]})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(workload, args.cpu_budget)

    metric = "2:4 sparse GEMM effective TFLOP/s + speedup vs dense GEMM; compress GB/s"
    result = {
        "metric": metric, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[dt], "data": "synthetic",
        "config": {"workload": workload, "shapes_NK": w["shapes"], "M": w["ms"], "dtype": DTYPE_NAME[dt],
                   "out_dtype": "f32" if out == inputs.F32 else DTYPE_NAME[out],
                   "cache": "cold (1 GiB read before each kernel)" if cold else "warm",
                   "seeds": "10000*c + 100*s + 10*t + j"},
        "speedup_vs_dense": round(speedup, 3),
        "compress_GBps": round(compress_gbps, 1),
        "compress_hbm_frac": round(compress_gbps / HBM_PEAK_GBPS, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "cases": rows,
        "tactics": tactics,
        "versions": {"torch": torch.__version__, "hip": torch.version.hip, "lib": sp.version()},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
