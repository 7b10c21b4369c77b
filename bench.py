"""Benchmark of the 2:4 sparse GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all]

A step is one pass of the whole hot path over a workload's synthetic, seeded
operands: for every weight shape, prune+compress the weight (or, for the
online workloads, the activation), decompress it (the dense pruned weight the
fallback uses), then for every M the sparse GEMM and the dense GEMM on the
same shapes.  Each of these runs as a chain of launches (the same count for
every case, about 1.5 ms of work for the fastest) captured in a HIP graph and
timed with HIP events on the stream it runs on (time per launch = chain time
/ launches).  HBM-bound workloads run "cold": the launches of a chain cycle
through copies of the weights totalling 640 MiB, so every launch reads its
operands from HBM as successive layers do; compute-bound ones run warm on one
copy.  After the timed steps the per-shape tactic (sparse iff faster) is
selected, the vendor dense GEMM (torch.mm, hipBLASLt) is timed on the bf16
shapes in chains like the library's, and the CPU oracle is timed on the host
cores.  On the bf16 workloads, whose four shapes are the projections of a
Llama-3-8B-like block, the tactic records also give the layer-level audit
manifest of 32 such blocks per M (its metrics in the line; --manifest-dir
writes it whole), once against the library's dense GEMM and once with the
same decision rule against the vendor dense GEMM ("audit_vs_vendor_dense":
sparse only where it beats both).

With no --workload (or --workload all) every workload runs in this process:
prefill first, the headline (its K timed steps after W warmup steps set
value, ms_per_step, roofline and cpu_baseline), then each other workload with
the same step counts as its own record under "workloads".  One JSON line is
printed.

--counter-pass runs each chain eagerly (no HIP graph) with at most a few
launches per chain, for rocprofv3 counter collection.

Workloads: tiny | decode | prefill | fp8 | int8 | online | online_fp8 | online_int8 | hybrid | ksplit
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
from semi_structured_sparse_sp24_amd import audit, inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
# published MI355X dense peaks (int8 in TOP/s), and twice that for 2:4, counted dense-equivalent
SPARSE_PEAK_TFLOPS = {inputs.BF16: 5033.0, inputs.F16: 5033.0, inputs.E4M3: 10066.0, inputs.I8: 10066.0}
DENSE_PEAK_TFLOPS = {inputs.BF16: 2516.0, inputs.F16: 2516.0, inputs.E4M3: 5033.0, inputs.I8: 5033.0}
DTYPE_NAME = {inputs.F16: "f16", inputs.BF16: "bf16", inputs.E4M3: "e4m3", inputs.I8: "i8"}
TORCH = {inputs.F16: torch.float16, inputs.BF16: torch.bfloat16, inputs.E4M3: torch.float8_e4m3fn,
         inputs.I8: torch.int8}


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


def hybrid_gemm_bytes(M, NS, ND, K, eb, out_eb):
    """Compressed rows (values + meta) + dense rows + X + the whole output."""
    return NS * K * eb // 2 + NS * K // 8 + ND * K * eb + M * K * eb + M * (NS + ND) * out_eb


def ksplit_gemm_bytes(M, N, KS, K, eb, out_eb):
    """The 2:4 K range (values + meta) + the dense K range of W + X + the output."""
    return N * KS * eb // 2 + N * KS // 8 + N * (K - KS) * eb + M * K * eb + M * N * out_eb


def compress_bytes(R, K, eb):
    return R * K * eb + R * K * eb // 2 + R * K // 8


def case_peak_tflops(workload, c, dt):
    """Dense-equivalent MFMA peak of one case: the 2:4 peak, or for the hybrids the rate at which
    their mix of 2:4 work (at the sparse rate) and dense work (at the dense rate) would run."""
    sp_peak, d_peak = SPARSE_PEAK_TFLOPS[dt], DENSE_PEAK_TFLOPS[dt]
    if workload == HYBRID:
        return (c["NS"] + c["ND"]) / (c["NS"] / sp_peak + c["ND"] / d_peak)
    if workload == KSPLIT:
        return c["K"] / (c["KS"] / sp_peak + c["KD"] / d_peak)
    return sp_peak


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


# Cold protocol for HBM-bound kernels: consecutive launches of a chain cycle through this many bytes
# of distinct operand copies, more than twice the 32 MB of L2 plus the 256 MB Infinity Cache, so that
# every launch reads its weights from HBM -- as the layers of a decode step do.  Warm kernels re-run
# on one copy.
COLD_BYTES = 640 << 20
ONLINE = ("online", "online_fp8", "online_int8")   # the activation is the compressed operand, compressed every call
# the activation arrives in bf16 and each side quantizes it itself: fused with the prune for the sparse
# side, plain for the dense side
QUANT_ONLINE = ("online_fp8", "online_int8")


def quantizers(workload):
    """(fused quantize + prune + compress, plain quantize) of a quantized online workload."""
    if workload == "online_int8":
        return sp.quantize_i8_prune_compress, sp.quantize_i8
    return sp.quantize_prune_compress, sp.quantize_e4m3


def oracle_quantizer(workload):
    """The oracle's fused quantize + prune + compress of a quantized online workload."""
    import oracle
    return oracle.quantize_i8_prune_compress if workload == "online_int8" else oracle.quantize_prune_compress
HYBRID = "hybrid"                   # weight rows split: 2:4 rows and dense rows in one launch
KSPLIT = "ksplit"                   # weight K range split: a 2:4 range and a dense range, one launch
MAX_COPIES = 64
# The shortest chain of a workload runs for about this long, so that the fixed cost of starting a
# graph (~20 us) stays a small part of the bracketed time.  Every GEMM chain of a workload has the
# same length (and every compress chain likewise): a step holds one launch of each case, so the
# per-launch averages of a kernel -- and the profiler's, over the same launches -- weight the cases
# equally, as one step does.  (Chain i of a cold case uses copy i % copies; a copy is reused only
# after every other copy, more than 640 MiB later.)
CHAIN_US = 1500.0


CHAIN_CAP = None   # the counter pass caps every chain at this many launches


def chain_length(est_us_list):
    """Launches per chain for a set of cases: CHAIN_US of work for the fastest, 8 to 256."""
    n = int(min(256, max(8, -(-CHAIN_US // max(min(est_us_list), 1.0)))))
    return n if CHAIN_CAP is None else min(n, CHAIN_CAP)


def est_us(nbytes, flops):
    """Rough duration of one launch (4 TB/s, 1 PFLOP/s, 2 us fixed) used only to size chains."""
    return max(nbytes / 4e6, flops / 1e9) + 2.0


def n_copies(compressed_bytes, cold):
    if not cold:
        return 1
    return int(min(MAX_COPIES, max(2, -(-COLD_BYTES // compressed_bytes))))


def build_cases(workload, cold):
    w = inputs.WORKLOADS[workload]
    dt, out = w["dtype"], w["out"]
    eb = inputs.ELEM_BYTES[dt]
    ytype = TORCH[out] if out in TORCH else torch.float32
    cases = []
    for s, (N, K) in enumerate(w["shapes"]):
        wb, sw = inputs.weight(workload, s)
        W0 = dev(wb, dt)
        shape = {"s": s, "N": N, "K": K, "sw": None if sw is None else torch.from_numpy(sw).cuda(), "ms": []}
        NS, KS = N, K
        if workload == HYBRID:
            # the first NS rows go 2:4, the rest stay dense; the dense baseline runs the same weight
            # (the pruned rows and the dense rows) through the dense GEMM
            NS, ND = inputs.hybrid_split(N)
            shape.update(NS=NS, ND=ND, Wd=W0[NS:].contiguous())
            W0 = W0[:NS].contiguous()
        if workload == KSPLIT:
            # the first KS columns of every row go 2:4, the rest stay dense; the dense baseline runs the
            # same weight (the pruned range and the dense range) through the dense GEMM
            KS, KD = inputs.ksplit_split(K)
            shape.update(KS=KS, KD=KD, Wd=W0[:, KS:].contiguous())
            W0 = W0[:, :KS].contiguous()
        nc = 1 if workload in ONLINE else n_copies(NS * KS * eb // 2 + NS * KS // 8, cold)
        copies = []
        for i in range(nc):
            W = W0 if i == 0 else W0.clone()
            v, m = sp.prune_compress(W)
            copies.append({"W": W, "v": v, "m": m, "Wp": sp.decompress(v, m, KS)})
        shape["copies"] = copies
        if workload == HYBRID:
            shape["Wfull"] = torch.cat([copies[0]["Wp"], shape["Wd"]]).contiguous()
        if workload == KSPLIT:
            shape["Wfull"] = torch.cat([copies[0]["Wp"], shape["Wd"]], dim=1).contiguous()
        for j, M in enumerate(w["ms"]):
            xb, sx = inputs.activation(workload, s, j)
            X = dev(xb, w.get("act", dt))
            item = {"j": j, "M": M, "X": X, "sx": None if sx is None else torch.from_numpy(sx).cuda(),
                    "Y": torch.empty((M, N), dtype=ytype, device="cuda"),
                    "Yd": torch.empty((M, N), dtype=ytype, device="cuda")}
            if workload in ONLINE:
                item["xv"] = torch.empty((M, K // 2), dtype=TORCH[dt], device="cuda")
                item["xm"] = torch.empty((M, (K + 31) // 32), dtype=torch.int32, device="cuda")
            if workload == HYBRID:
                item["Ys"] = torch.empty((M, shape["NS"]), dtype=ytype, device="cuda")
                item["Ydd"] = torch.empty((M, shape["ND"]), dtype=ytype, device="cuda")
            if workload in QUANT_ONLINE:
                # each side quantizes the bf16 activation itself: fused with the prune for the
                # sparse side, plain for the dense side
                item["xs"] = torch.empty(M, dtype=torch.float32, device="cuda")
                item["xq"] = torch.empty((M, K), dtype=TORCH[dt], device="cuda")
                item["xqs"] = torch.empty(M, dtype=torch.float32, device="cuda")
            shape["ms"].append(item)
        cases.append(shape)
    torch.cuda.synchronize()
    return cases


def chains(workload, cases):
    """The step as an ordered list of (key, launches, fn): fn(i) issues launch i of the chain."""
    w = inputs.WORKLOADS[workload]
    eb = inputs.ELEM_BYTES[w["dtype"]]
    Lg = chain_length([est_us((c["N"] * c["K"] + it["M"] * c["K"]) * eb, 2.0 * it["M"] * c["N"] * c["K"])
                       for c in cases for it in c["ms"]])
    if workload in ONLINE:
        Lc = chain_length([est_us(it["M"] * c["K"] * 2 * 1.625, 0) for c in cases for it in c["ms"]])
    else:
        Lc = chain_length([est_us(c["N"] * c["K"] * eb * 1.625, 0) for c in cases])
    out = []
    for c in cases:
        N, K, cp = c["N"], c["K"], c["copies"]
        pick = lambda i, cp=cp: cp[i % len(cp)]
        if workload not in ONLINE:
            Kc = c.get("KS", K)
            out.append((("compress", c["s"]), Lc,
                        lambda i, pick=pick: sp.prune_compress(pick(i)["W"], values=pick(i)["v"], meta=pick(i)["m"])))
            out.append((("decompress", c["s"]), Lc,
                        lambda i, pick=pick, Kc=Kc: sp.decompress(pick(i)["v"], pick(i)["m"], Kc, out=pick(i)["Wp"])))
        for it in c["ms"]:
            M, key = it["M"], (c["s"], it["j"])
            if workload in QUANT_ONLINE:
                W, sw = cp[0]["W"], c["sw"]
                fused, plain = quantizers(workload)
                out.append((("compress",) + key, Lc,
                            lambda i, it=it, fused=fused: fused(it["X"], values=it["xv"], meta=it["xm"],
                                                                scales=it["xs"])))
                out.append((("sparse",) + key, Lg,
                            lambda i, it=it, W=W, sw=sw, M=M, N=N, K=K:
                            sp.sp24_gemm(sp.SPARSE_X, it["xv"], it["xm"], W, M, N, K, scale_x=it["xs"],
                                         scale_w=sw, out=it["Y"])))
                out.append((("prep",) + key, Lc,
                            lambda i, it=it, plain=plain: plain(it["X"], out=it["xq"], scales=it["xqs"])))
                out.append((("dense",) + key, Lg,
                            lambda i, it=it, W=W, sw=sw: sp.dense_gemm(it["xq"], W, scale_x=it["xqs"], scale_w=sw,
                                                                       out=it["Yd"])))
                continue
            if workload == HYBRID:
                # one launch for both regions; against the dense GEMM on the whole weight, and against
                # the same split as two launches (sparse GEMM on the 2:4 rows, dense GEMM on the rest)
                NS, ND, Wd, Wf = c["NS"], c["ND"], c["Wd"], c["Wfull"]
                out.append((("sparse",) + key, Lg,
                            lambda i, it=it, pick=pick, Wd=Wd, NS=NS, ND=ND:
                            sp.hybrid_gemm(pick(i)["v"], pick(i)["m"], Wd, it["X"], NS, ND, out=it["Y"])))
                out.append((("dense",) + key, Lg, lambda i, it=it, Wf=Wf: sp.dense_gemm(it["X"], Wf, out=it["Yd"])))

                def split(i, it=it, pick=pick, Wd=Wd, M=M, NS=NS, K=K):
                    sp.sp24_gemm(sp.SPARSE_W, pick(i)["v"], pick(i)["m"], it["X"], M, NS, K, out=it["Ys"])
                    sp.dense_gemm(it["X"], Wd, out=it["Ydd"])
                out.append((("split",) + key, Lg, split))
                continue
            if workload == KSPLIT:
                # one launch for both K ranges, against the dense GEMM on the whole weight
                KS, Wd, Wf = c["KS"], c["Wd"], c["Wfull"]
                out.append((("sparse",) + key, Lg,
                            lambda i, it=it, pick=pick, Wd=Wd, N=N, KS=KS:
                            sp.ksplit_gemm(pick(i)["v"], pick(i)["m"], Wd, it["X"], N, KS, out=it["Y"])))
                out.append((("dense",) + key, Lg, lambda i, it=it, Wf=Wf: sp.dense_gemm(it["X"], Wf, out=it["Yd"])))
                continue
            if workload == "online":
                # the activation is the sparse operand: prune+compress it on every call
                W = cp[0]["W"]
                out.append((("compress",) + key, Lc,
                            lambda i, it=it: sp.prune_compress(it["X"], values=it["xv"], meta=it["xm"])))
                out.append((("sparse",) + key, Lg,
                            lambda i, it=it, W=W, M=M, N=N, K=K:
                            sp.sp24_gemm(sp.SPARSE_X, it["xv"], it["xm"], W, M, N, K, out=it["Y"])))
                out.append((("dense",) + key, Lg, lambda i, it=it, W=W: sp.dense_gemm(it["X"], W, out=it["Yd"])))
                continue
            out.append((("sparse",) + key, Lg,
                        lambda i, it=it, pick=pick, M=M, N=N, K=K, c=c:
                        sp.sp24_gemm(sp.SPARSE_W, pick(i)["v"], pick(i)["m"], it["X"], M, N, K,
                                     scale_x=it["sx"], scale_w=c["sw"], out=it["Y"])))
            out.append((("dense",) + key, Lg,
                        lambda i, it=it, pick=pick, c=c:
                        sp.dense_gemm(it["X"], pick(i)["Wp"], scale_x=it["sx"], scale_w=c["sw"], out=it["Yd"])))
    return out


class Runner:
    """Each chain is captured once in a HIP graph (so launches follow each other with no host gap)
    and replayed between two HIP events on the stream it was captured for; the per-launch time is
    the bracketed time over the chain's length.  With eager=True (the counter pass) the chains are
    launched one call at a time instead, with no graph."""

    def __init__(self, items, eager=False):
        self.items = items
        self.eager = eager
        for _, n, fn in items:          # eager pass: loads every code object before capture
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        self.length = {key: n for key, n, _ in items}
        self.graphs = []
        if not eager:
            for _, n, fn in items:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n):
                        fn(i)
                self.graphs.append(g)
        torch.cuda.synchronize()
        self.pending = []

    def step(self):
        for idx, (key, n, fn) in enumerate(self.items):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            if self.eager:
                for i in range(n):
                    fn(i)
            else:
                self.graphs[idx].replay()
            b.record()
            self.pending.append((key, n, a, b))

    def release(self):
        self.graphs = []
        self.items = []

    def collect(self):
        torch.cuda.synchronize()
        out = {}
        for key, n, a, b in self.pending:
            out.setdefault(key, []).append(a.elapsed_time(b) * 1e3 / n)   # microseconds per launch
        self.pending = []
        return out


def layer_audit(workload, w, records, manifest_dir, tag="",
                time_note="each layer at its selected path's warm median from the tactic record"):
    """The layer-level manifest of a Llama-3-8B-like stack (32 blocks of the four projections
    whose shapes the bf16 workloads time), one per M, from the tactic records of this run:
    its metrics go into the bench line, the whole manifest into manifest_dir if given."""
    shapes = sorted(tuple(x) for x in w["shapes"])
    if not records or shapes != sorted((N, K) for _, N, K in audit.LLAMA3_8B_BLOCK):
        return None
    if any((N, K, M) not in records for M in w["ms"] for _, N, K in audit.LLAMA3_8B_BLOCK):
        return None
    revision = audit.synthetic_revision(f"{workload}:{w['shapes']}:10000*c + 100*s + 10*t + j")
    out = {"model": f"Llama-3-8B-like: {audit.LLAMA3_8B_BLOCKS} blocks x (qkv, o, gate_up, down)",
           "time": time_note + "; no time outside these layers (attention, norms) is counted",
           "per_M": {}}
    for M in w["ms"]:
        by_shape = {(N, K): records[(N, K, M)] for _, N, K in audit.LLAMA3_8B_BLOCK}
        man = audit.block_manifest(by_shape, revision, extra={
            "workload": {"name": workload, "tokens_per_call": M},
            "runtime": {"torch": torch.__version__, "hip": torch.version.hip, "lib": sp.version()}})
        out["per_M"][str(M)] = man["metrics"]
        if manifest_dir:
            os.makedirs(manifest_dir, exist_ok=True)
            name = f"manifest_{workload}_M{M}" + (f"_{tag}" if tag else "") + ".json"
            with open(os.path.join(manifest_dir, name), "w") as f:
                json.dump(man, f, indent=1)
    return out


def cpu_info():
    """The host the CPU baseline runs on: model name, cores this process may run on, OpenMP threads."""
    import oracle

    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "omp_threads": oracle.num_threads()}


def compressed_operands(workload):
    """(name, dtype, bits) of every operand the workload prunes and compresses: its weights (the 2:4
    rows of a hybrid weight, the 2:4 K range of a K-split one), or its activations when they are
    the compressed operand."""
    w = inputs.WORKLOADS[workload]
    dt = w["dtype"]
    out = []
    for s, (N, K) in enumerate(w["shapes"]):
        if workload in ONLINE:
            for j, M in enumerate(w["ms"]):
                xb, _ = inputs.activation(workload, s, j)
                out.append((f"X({M},{K})", w.get("act", dt), xb))
            continue
        wb, _ = inputs.weight(workload, s)
        if workload == HYBRID:
            NS, _ = inputs.hybrid_split(N)
            wb = wb[:NS]
        elif workload == KSPLIT:
            KS, _ = inputs.ksplit_split(K)
            wb = np.ascontiguousarray(wb[:, :KS])
        out.append((f"W{wb.shape}", dt, wb))
    return out


def cpu_compress(workload, budget_s):
    """The oracle's prune+compress (the fused quantize + prune + compress for the quantized online
    workloads) on the full
    operands of the workload, with every OpenMP thread and with one, in GB/s of algorithmic bytes."""
    import oracle

    threads = oracle.num_threads()
    res = {}
    for n in (threads, 1):
        oracle.set_num_threads(n)
        nbytes, secs, names = 0.0, 0.0, []
        for name, dt, bits in compressed_operands(workload):
            R, K = bits.shape
            t0 = time.perf_counter()
            if workload in QUANT_ONLINE:
                oracle_quantizer(workload)(dt, bits)
                nbytes += R * K * 2 + R * K // 2 + R * K // 8 + 4 * R
            else:
                oracle.prune_compress(dt, bits)
                nbytes += compress_bytes(R, K, inputs.ELEM_BYTES[dt])
            secs += time.perf_counter() - t0
            names.append(name)
            if secs >= budget_s:
                break
        res["GBps_all_threads" if n == threads else "GBps_one_thread"] = round(nbytes / secs / 1e9, 3)
        res["operands"] = " ".join(names)
    oracle.set_num_threads(threads)
    res["threads"] = threads
    return res


def cpu_baseline(workload, budget_s):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: its GEMMs (fp64 on the decompressed weight) over the
    workload's (shape, M) cases, rows of M sampled when M is large, passes over
    the cases repeated until about budget_s seconds of GEMM time are spent;
    and its prune+compress on the full operands, with all threads and with one."""
    import oracle

    w = inputs.WORKLOADS[workload]
    dt = w["dtype"]
    prepared = []
    for s, (N, K) in enumerate(w["shapes"]):
        wb, sw = inputs.weight(workload, s)
        wv = wm = None
        if workload == HYBRID:
            NS, _ = inputs.hybrid_split(N)
            wv, wm = oracle.prune_compress(dt, wb[:NS])
        elif workload == KSPLIT:
            KS, _ = inputs.ksplit_split(K)
            wv, wm = oracle.prune_compress(dt, np.ascontiguousarray(wb[:, :KS]))
        elif workload not in ONLINE:
            wv, wm = oracle.prune_compress(dt, wb)
        for j, M in enumerate(w["ms"]):
            xb, sx = inputs.activation(workload, s, j)
            rows = M if M <= 64 else 16
            mrows = np.linspace(0, M - 1, rows).astype(np.int64)
            xv = xm = None
            if workload == "online":
                xv, xm = oracle.prune_compress(dt, xb)
            elif workload in QUANT_ONLINE:
                xv, xm, sx = oracle_quantizer(workload)(w["act"], xb)
            prepared.append((N, K, M, rows, mrows, wb, sw, wv, wm, xb, sx, xv, xm))
    flops = 0.0
    secs = 0.0
    calls = 0
    names = []
    while secs < budget_s:
        for (N, K, M, rows, mrows, wb, sw, wv, wm, xb, sx, xv, xm) in prepared:
            t0 = time.perf_counter()
            if workload in ONLINE:
                oracle.gemm(dt, M, N, K, x_vals=xv, x_meta=xm, w=wb, scale_x=sx, scale_w=sw, mrows=mrows)
            elif workload == HYBRID:
                NS, ND = inputs.hybrid_split(N)
                oracle.hybrid_gemm(dt, rows, NS, ND, K, x=xb[mrows], ws_vals=wv, ws_meta=wm, wd=wb[NS:])
            elif workload == KSPLIT:
                KS, _ = inputs.ksplit_split(K)
                oracle.ksplit_gemm(dt, rows, N, KS, K, x=xb[mrows], ws_vals=wv, ws_meta=wm,
                                   wd=np.ascontiguousarray(wb[:, KS:]))
            else:
                oracle.gemm(dt, M, N, K, x=xb, w_vals=wv, w_meta=wm, scale_x=sx, scale_w=sw, mrows=mrows)
            secs += time.perf_counter() - t0
            flops += 2.0 * rows * N * K
            calls += 1
            if len(names) < len(prepared):
                names.append(f"({N},{K})xM{M}" + ("" if rows == M else f"[{rows} rows]"))
            if secs >= budget_s:
                break
    out = {"value": flops / secs / 1e12 if secs > 0 else None, "unit": "TFLOP/s",
           "cores": oracle.num_threads(), "kind": "oracle",
           "sample": "oracle fp64 GEMM on the decompressed operand over the cases " + " ".join(names) +
                     f": {calls} calls, {secs:.1f} s of GEMM time; rows of M > 64 sampled (16 evenly spaced), "
                     "TFLOP/s counted on the rows computed"}
    out.update(cpu_info())
    out["compress"] = cpu_compress(workload, max(2.0, budget_s / 2))
    return out


def vendor_dense(workload, cases, steps=3):
    """The vendor dense GEMM (torch.mm, hipBLASLt) on the same dense pruned weights and
    activations, timed as the library's chains are: the dense side of the vendor-aware tactic,
    not part of the step.  bf16 weight-compressed workloads only; per-launch microseconds of each
    step (the first, untimed, dropped) by case."""
    if workload not in ("prefill", "decode"):
        return None
    w = inputs.WORKLOADS[workload]
    eb = inputs.ELEM_BYTES[w["dtype"]]
    L = chain_length([est_us((c["N"] * c["K"] + it["M"] * c["K"]) * eb, 2.0 * it["M"] * c["N"] * c["K"])
                      for c in cases for it in c["ms"]])
    items = []
    for c in cases:
        cp = c["copies"]
        for it in c["ms"]:
            items.append((("vendor", c["s"], it["j"]), L,
                          lambda i, it=it, cp=cp: torch.mm(it["X"], cp[i % len(cp)]["Wp"].t(), out=it["Yd"])))
    r = Runner(items)
    for _ in range(steps + 1):
        r.step()
    t = r.collect()
    r.release()
    return {(key[1], key[2]): [float(x) for x in v[1:]] for key, v in t.items()}


def measure(workload, args, steps, warmup, cpu_budget, eager=False):
    """Runs one workload: warmup + timed steps, then the tactic, the vendor context and the CPU
    baseline.  Returns the record and the wall time of the timed steps."""
    w = inputs.WORKLOADS[workload]
    dt, out = w["dtype"], w["out"]
    eb, out_eb = inputs.ELEM_BYTES[dt], inputs.ELEM_BYTES[out]
    cold = (workload in ("decode", "fp8", "int8", "tiny")) if args.cold == "auto" else args.cold == "on"
    scales = dt in (inputs.E4M3, inputs.I8)

    cases = build_cases(workload, cold)
    runner = Runner(chains(workload, cases), eager=eager)
    for _ in range(warmup):
        runner.step()
    runner.collect()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        runner.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = runner.collect()
    lengths = dict(runner.length)
    runner.release()

    if args.copy_calibration_mib:
        # a kernel that reads and writes exactly this many bytes (an elementwise negation, which
        # a DMA engine cannot take over as it may a plain copy): the yardstick for the byte counters
        n = args.copy_calibration_mib << 18
        a = torch.ones(n, dtype=torch.int32, device="cuda")
        b = torch.empty(n, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    vendor = None if (eager or args.no_vendor) else vendor_dense(workload, cases)

    # ---------------------------------------------------------------- per-case table
    rows = []
    vendor_records = {}
    tot = {"sparse_t": 0.0, "dense_t": 0.0, "flops": 0.0, "sparse_bytes": 0.0, "compress_t": 0.0,
           "compress_bytes": 0.0, "sparse_launches": 0}
    for c in cases:
        N, K = c["N"], c["K"]
        for it in c["ms"]:
            M = it["M"]
            key = (c["s"], it["j"])
            ts = times[("sparse",) + key]
            td = times[("dense",) + key]
            sparse_rows = M if workload in ONLINE else N
            if workload == HYBRID:
                sb = hybrid_gemm_bytes(M, c["NS"], c["ND"], K, eb, out_eb)
            elif workload == KSPLIT:
                sb = ksplit_gemm_bytes(M, N, c["KS"], K, eb, out_eb)
            else:
                sb = sparse_gemm_bytes(M, N, K, eb, out_eb, sparse_rows, scales)
            db = dense_gemm_bytes(M, N, K, eb, out_eb, scales)
            fl = 2.0 * M * N * K
            tsm, tdm = float(np.median(ts)), float(np.median(td))
            case_peak = case_peak_tflops(workload, c, dt)
            row = {"N": N, "K": K, "M": M, "t_sparse_us": round(tsm, 2), "t_dense_us": round(tdm, 2),
                   "speedup": round(tdm / tsm, 3),
                   "sparse_tflops": round(fl / tsm / 1e6, 1), "dense_tflops": round(fl / tdm / 1e6, 1),
                   "sparse_GBps": round(sb / tsm / 1e3, 1), "dense_GBps": round(db / tdm / 1e3, 1),
                   "sparse_hbm_frac": round(sb / tsm / 1e3 / HBM_PEAK_GBPS, 3),
                   "sparse_mfma_frac": round(fl / tsm / 1e6 / case_peak, 3),
                   # the case's own roofline: min(MFMA peak, arithmetic intensity x HBM peak), which at
                   # the ridge (prefill M = 512) is below both peaks
                   "sparse_attainable_frac": round(
                       (fl / tsm / 1e6) / min(case_peak, fl / sb * HBM_PEAK_GBPS / 1e3), 3),
                   "t_sparse_p10_us": round(float(np.percentile(ts, 10)), 2),
                   "t_sparse_p90_us": round(float(np.percentile(ts, 90)), 2)}
            if vendor is not None:
                tv = float(np.median(vendor[key]))
                # the pages' rule with the fastest dense GEMM on this part as the dense side: the
                # sparse path is selected only where it beats the vendor's dense GEMM as well
                vrec = sp.tactic_decide(True, [float(x) for x in ts], vendor[key])
                if vrec["selected"] == "dense":
                    vrec["kernel"] = "hipBLASLt (torch.mm)"
                vendor_records[(N, K, M)] = vrec
                row.update(t_vendor_dense_us=round(tv, 2), speedup_vs_vendor_dense=round(tv / tsm, 3),
                           own_dense_vs_vendor=round(tdm / tv, 3), selected_vs_vendor=vrec["selected"])
            if workload == HYBRID:
                tsp = float(np.median(times[("split",) + key]))
                row.update(N_s=c["NS"], N_d=c["ND"], t_two_launch_us=round(tsp, 2),
                           speedup_vs_two_launch=round(tsp / tsm, 3))
            if workload == KSPLIT:
                row.update(K_s=c["KS"], K_d=c["KD"])
            if workload in ONLINE:
                tc = float(np.median(times[("compress",) + key]))
                tp = float(np.median(times[("prep",) + key])) if workload in QUANT_ONLINE else 0.0
                row["t_compress_us"] = round(tc, 2)
                if workload in QUANT_ONLINE:
                    row["t_dense_quantize_us"] = round(tp, 2)
                row["speedup_incl_compress"] = round((tp + tdm) / (tc + tsm), 3)
                tot["compress_t"] += sum(times[("compress",) + key])
                cb = (M * K * 2 + M * K // 2 + M * K // 8 + 4 * M) if workload in QUANT_ONLINE \
                    else compress_bytes(M, K, eb)
                tot["compress_bytes"] += cb * len(times[("compress",) + key])
            rows.append(row)
            tot["sparse_t"] += sum(ts)
            tot["dense_t"] += sum(td)
            tot["flops"] += fl * len(ts)
            tot["sparse_bytes"] += sb * len(ts)
            tot["sparse_launches"] += len(ts)
        if workload not in ONLINE:
            tcs = times[("compress", c["s"])]
            tot["compress_t"] += sum(tcs)
            R = c.get("NS", N)
            Kc = c.get("KS", K)
            tot["compress_bytes"] += compress_bytes(R, Kc, eb) * len(tcs)

    value = tot["flops"] / tot["sparse_t"] / 1e6                    # TFLOP/s (dense-equivalent)
    speedup = tot["dense_t"] / tot["sparse_t"]
    compress_gbps = tot["compress_bytes"] / tot["compress_t"] / 1e3

    # roofline of the dominant kernel: the sparse GEMM kernel (by name, as the dispatch picks it per
    # shape) with the largest share of the step's sparse GEMM time; achieved = its algorithmic bytes
    # (HBM-bound decode) or flops (MFMA-bound prefill) per launch / its mean launch duration, over
    # all its launches (every case of the kernel has the same number of launches)
    per_kernel = {}
    for c in cases:
        for it in c["ms"]:
            M, N, K = it["M"], c["N"], c["K"]
            which = sp.SPARSE_X if workload in ONLINE else sp.SPARSE_W
            if workload == HYBRID:
                name = sp.hybrid_kernel(TORCH[dt], it["Y"].dtype, M, c["NS"], c["ND"], K)
            elif workload == KSPLIT:
                name = sp.ksplit_kernel(TORCH[dt], it["Y"].dtype, M, N, c["KS"], K)
            else:
                name = sp.gemm_kernel(True, which, TORCH[dt], it["Y"].dtype, M, N, K)
            key = ("sparse", c["s"], it["j"])
            ts, L = times[key], lengths[key]       # per-launch means of each step; chain length
            sparse_rows = M if workload in ONLINE else N
            k = per_kernel.setdefault(name, {"t": 0.0, "n": 0, "bytes": 0.0, "flops": 0.0, "t_peak": 0.0})
            # weighted by launches, as a profiler's per-kernel average is
            k["t"] += sum(ts) * L
            k["n"] += len(ts) * L
            if workload == HYBRID:
                k["bytes"] += hybrid_gemm_bytes(M, c["NS"], c["ND"], K, eb, out_eb) * len(ts) * L
            elif workload == KSPLIT:
                k["bytes"] += ksplit_gemm_bytes(M, N, c["KS"], K, eb, out_eb) * len(ts) * L
            else:
                k["bytes"] += sparse_gemm_bytes(M, N, K, eb, out_eb, sparse_rows, scales) * len(ts) * L
            # time at peak (the hybrids' dense parts at the dense rate)
            k["t_peak"] += 2.0 * M * N * K / case_peak_tflops(workload, c, dt) / 1e6 * len(ts) * L
            k["flops"] += 2.0 * M * N * K * len(ts) * L
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
        # the kernel's own peak in dense-equivalent flops (for the hybrids, the rate at which their mix
        # of 2:4 and dense work would run with every instruction at peak)
        peak = round(k["flops"] / k["t_peak"] / 1e6, 1)
        achieved = k["flops"] / k["t"] / 1e6
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_per_launch(kname, workload),
                "kernel": kname, "launches": k["n"], "flops_per_launch": round(k["flops"] / k["n"]),
                "bytes_per_launch": round(k["bytes"] / k["n"]), "avg_launch_us": round(avg_us, 3)}
    if hbm_bound and not eager:
        roof.update(copy_reference())
        roof["frac_of_measured_copy"] = round(achieved / roof["measured_copy_GBps"], 4)
    all_t = sum(v["t"] for v in per_kernel.values())
    roof["kernels"] = {n: {"launches": v["n"], "avg_launch_us": round(v["t"] / v["n"], 3),
                           "share": round(v["t"] / all_t, 3)} for n, v in per_kernel.items()}

    tactics = []
    records = {}
    if not (args.no_tactic or eager) and workload not in (HYBRID, KSPLIT):
        for c in cases:
            for it in c["ms"]:
                M, N, K = it["M"], c["N"], c["K"]
                if workload in QUANT_ONLINE:
                    # both sides quantize; the tactic compares the rest: prune+compress of the codes
                    # and the sparse GEMM against the dense GEMM on the codes
                    rec = sp.select_tactic(sp.SPARSE_X, it["xv"], it["xm"], c["copies"][0]["W"], it["xq"], M, N, K,
                                           scale_x=it["xqs"], scale_w=c["sw"], y_scratch=it["Y"], warmup=3,
                                           reps=10)
                elif workload == "online":
                    rec = sp.select_tactic(sp.SPARSE_X, it["xv"], it["xm"], c["copies"][0]["W"], it["X"], M, N, K,
                                           y_scratch=it["Y"], warmup=3, reps=10)
                else:
                    rec = sp.select_tactic(sp.SPARSE_W, c["copies"][0]["v"], c["copies"][0]["m"], it["X"],
                                           c["copies"][0]["Wp"], M, N, K, scale_x=it["sx"], scale_w=c["sw"],
                                           y_scratch=it["Y"], warmup=3, reps=10)
                tactics.append({"N": N, "K": K, "M": M, "selected": rec["selected"], "ratio": round(rec["ratio"], 3),
                                "reason": rec["reason"], "kernel": rec["kernel"]})
                records[(N, K, M)] = rec
    audit_summary = layer_audit(workload, w, records, args.manifest_dir)
    audit_vendor = layer_audit(workload, w, vendor_records, args.manifest_dir, tag="vs_vendor",
                               time_note="each layer at its selected path's median per-launch time in this "
                                         "run's bench chains (the step's cache mode)")
    if audit_vendor is not None:
        audit_vendor["dense_side"] = "hipBLASLt through torch.mm on the same pruned weights"
    del cases
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    cpu = None
    if not (args.no_cpu_baseline or eager):
        cpu = cpu_baseline(workload, cpu_budget)

    result = {
        "value": round(value, 3), "unit": "TFLOP/s", "dtype": DTYPE_NAME[dt], "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall / max(steps, 1) * 1e3, 3),
        "config": {"workload": workload, "shapes_NK": w["shapes"], "M": w["ms"], "dtype": DTYPE_NAME[dt],
                   "out_dtype": "f32" if out == inputs.F32 else DTYPE_NAME[out],
                   "cache": "cold (launches cycle through 640 MiB of weight copies)" if cold else "warm",
                   "seeds": "10000*c + 100*s + 10*t + j",
                   "timing": "eager launches (counter pass)" if eager else "HIP graph chains"},
        "speedup_vs_dense": round(speedup, 3),
        "compress_GBps": round(compress_gbps, 1),
        "compress_hbm_frac": round(compress_gbps / HBM_PEAK_GBPS, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "cases": rows,
        "tactics": tactics,
        "audit": audit_summary,
        "audit_vs_vendor_dense": audit_vendor,
    }
    return result, wall


_COPY = {}


def copy_reference():
    """A bandwidth this part reaches: an elementwise negation over 512 MiB (reads and writes 512
    MiB), timed once per process after the first HBM-bound workload's steps."""
    if not _COPY:
        a = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(2):
            torch.neg(a, out=b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            torch.neg(a, out=b)
        e1.record()
        torch.cuda.synchronize()
        _COPY["measured_copy_GBps"] = round(2 * a.numel() * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del a, b
        torch.cuda.empty_cache()
    return dict(_COPY)


def compact(rec):
    """A non-headline workload's record in the line: the per-case table kept to its main columns."""
    keep = ("N", "K", "M", "N_s", "N_d", "K_s", "K_d", "t_sparse_us", "t_dense_us", "speedup", "sparse_tflops",
            "sparse_GBps", "sparse_hbm_frac", "sparse_mfma_frac", "t_compress_us", "speedup_incl_compress",
            "t_two_launch_us", "t_vendor_dense_us", "selected_vs_vendor")
    out = dict(rec)
    out["cases"] = [{k: v for k, v in r.items() if k in keep} for r in rec["cases"]]
    out["roofline"] = {k: v for k, v in rec["roofline"].items() if k != "kernels"}
    return out


ORDER = [n for n in ("prefill", "tiny", "decode", "fp8", "int8", "online", "online_fp8", "online_int8", "hybrid",
                    "ksplit")
         if n in inputs.WORKLOADS]


def main():
    global CHAIN_CAP
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=["all"] + list(inputs.WORKLOADS))
    ap.add_argument("--cold", choices=["auto", "on", "off"], default="auto")
    ap.add_argument("--cpu-budget", type=float, default=None,
                    help="seconds of oracle GEMM time per workload (default: 12 for the headline or a single "
                         "workload, 4 for each other workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tactic", action="store_true")
    ap.add_argument("--no-vendor", action="store_true", help="skip the hipBLASLt timing and the vendor-aware audit")
    ap.add_argument("--manifest-dir", default=None,
                    help="write the layer-level audit manifest of each M there (bf16 workloads)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (for counter calibration)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="launch every chain eagerly (no HIP graph), at most --chain-cap launches a chain, "
                         "and skip the tactic, vendor and CPU legs: the mode for rocprofv3 --pmc runs")
    ap.add_argument("--chain-cap", type=int, default=4)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path runs on a single MI355X, and sharding across GPUs is "
              "a design note only, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sp.lib()                                   # fails loudly if the HIP library is missing
    if args.counter_pass:
        CHAIN_CAP = args.chain_cap

    names = ORDER if args.workload == "all" else [args.workload]
    head = names[0]
    records = {}
    wall_head = None
    for name in names:
        budget = args.cpu_budget if args.cpu_budget is not None else (12.0 if name == head else 4.0)
        t0 = time.perf_counter()
        rec, wall = measure(name, args, args.steps, args.warmup, budget, eager=args.counter_pass)
        rec["wall_s"] = round(time.perf_counter() - t0, 1)
        records[name] = rec
        if name == head:
            wall_head = wall
        print(f"[bench] {name}: {rec['value']} TFLOP/s, roofline {rec['roofline']['frac']} of "
              f"{rec['roofline']['peak']} {rec['roofline']['unit']} ({rec['wall_s']} s)", file=sys.stderr,
              flush=True)

    h = records[head]
    metric = "2:4 sparse GEMM effective TFLOP/s + speedup vs dense GEMM; compress GB/s"
    result = {
        "metric": metric, "value": h["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_head / max(args.steps, 1) * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": h["dtype"],
        "data": "synthetic", "config": h["config"],
        "speedup_vs_dense": h["speedup_vs_dense"], "compress_GBps": h["compress_GBps"],
        "compress_hbm_frac": h["compress_hbm_frac"], "roofline": h["roofline"], "cpu_baseline": h["cpu_baseline"],
        "cases": h["cases"], "tactics": h["tactics"], "audit": h["audit"],
        "audit_vs_vendor_dense": h["audit_vs_vendor_dense"],
        "workloads": {n: compact(r) for n, r in records.items() if n != head},
        "versions": {"torch": torch.__version__, "hip": torch.version.hip, "lib": sp.version()},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
