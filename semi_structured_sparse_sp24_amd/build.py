"""Builds libsp24.so (HIP for gfx950) in-tree, next to this file.

Every .hip source under csrc/ is compiled with hipcc in parallel and linked
into one shared library that exports only the C ABI of include/sp24.h.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsp24.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "compress.hip", "quantize.hip", "gemm_sparse.hip", "gemm_sparse_big.hip",
           "gemm_dense.hip", "gemm_dense_big.hip"]

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    # packed fp32 ops stay off: the compiler must not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the large GEMM tiles fully unroll loops over 64 accumulator fragments per stage; the default
    # limit on pragma-requested unrolling would leave them partly rolled (accumulators on the stack)
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-I" + INCLUDE, "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that warning is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
