"""Host logic of bench.py (no GPU): the algorithmic byte counts and peaks the
roofline divides by, the staleness guard of the recorded traffic, the layer
audit's completeness check, and the one-GPU exit."""
import os
import subprocess
import sys

import pytest

import bench
from semi_structured_sparse_sp24_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_sparse_bytes_weight_compressed_bf16():
    # W (N x K) compressed: values N*K/2 elements of 2 bytes, metadata N*K/32 words of 4 bytes;
    # X (M x K) and Y (M x N) dense bf16
    M, N, K = 16, 4096, 4096
    values = N * (K // 2) * 2
    meta = N * (K // 32) * 4
    assert bench.sparse_gemm_bytes(M, N, K, 2, 2, N, False) == values + meta + M * K * 2 + M * N * 2


def test_sparse_bytes_activation_compressed_fp8_with_scales():
    # X (M x K) compressed e4m3, W (N x K) dense e4m3, bf16 output, one fp32 scale per row of each
    M, N, K = 4096, 28672, 4096
    values = M * (K // 2)
    meta = M * (K // 32) * 4
    assert bench.sparse_gemm_bytes(M, N, K, 1, 2, M, True) == \
        values + meta + N * K + M * N * 2 + 4 * (M + N)


def test_dense_hybrid_ksplit_and_compress_bytes():
    M, N, K = 2048, 4096, 4096
    assert bench.dense_gemm_bytes(M, N, K, 2, 2, False) == (M + N) * K * 2 + M * N * 2
    NS, ND = inputs.hybrid_split(N)
    assert NS + ND == N
    assert bench.hybrid_gemm_bytes(M, NS, ND, K, 2, 2) == \
        NS * K + NS * K // 8 + ND * K * 2 + M * K * 2 + M * N * 2
    KS, KD = inputs.ksplit_split(K)
    assert bench.ksplit_gemm_bytes(M, N, KS, K, 2, 2) == \
        N * KS + N * KS // 8 + N * KD * 2 + M * K * 2 + M * N * 2
    # the degenerate splits are the plain sparse and dense byte counts
    assert bench.ksplit_gemm_bytes(M, N, K, K, 2, 2) == bench.sparse_gemm_bytes(M, N, K, 2, 2, N, False)
    assert bench.ksplit_gemm_bytes(M, N, 0, K, 2, 2) == bench.dense_gemm_bytes(M, N, K, 2, 2, False)
    # compress reads the dense operand and writes values + metadata: 3.125 B per bf16 element
    assert bench.compress_bytes(N, K, 2) == N * K * 3.125


def test_case_peaks():
    bf = inputs.BF16
    assert bench.case_peak_tflops("prefill", {}, bf) == bench.SPARSE_PEAK_TFLOPS[bf]
    sp, de = bench.SPARSE_PEAK_TFLOPS[bf], bench.DENSE_PEAK_TFLOPS[bf]
    # all 2:4 or all dense reduce to the two peaks; a mix lies between them
    assert bench.case_peak_tflops("hybrid", {"NS": 4096, "ND": 0}, bf) == pytest.approx(sp)
    assert bench.case_peak_tflops("hybrid", {"NS": 0, "ND": 4096}, bf) == pytest.approx(de)
    mix = bench.case_peak_tflops("ksplit", {"K": 4096, "KS": 3072, "KD": 1024}, bf)
    # time at peak = 3072/sp + 1024/de per unit of the mix
    assert mix == pytest.approx(4096 / (3072 / sp + 1024 / de))
    assert de < mix < sp


def _fake_tree(tmp_path, digest):
    csrc = tmp_path / "semi_structured_sparse_sp24_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_bytes(b"kernel source\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.md").write_text(
        "| kernel | workload | source:sha256 | HBM bytes per launch |\n|---|---|---|---:|\n"
        f"| kern_a | wl | k.hip:{digest} | 12345 |\n")


def test_traffic_record_read_while_source_unchanged(tmp_path, monkeypatch):
    import hashlib
    digest = hashlib.sha256(b"kernel source\n").hexdigest()[:12]
    _fake_tree(tmp_path, digest)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch("kern_a", "wl") == 12345.0
    assert bench.traffic_per_launch("kern_a", "other") is None
    assert bench.traffic_per_launch("kern_b", "wl") is None


def test_traffic_record_stale_after_source_change(tmp_path, monkeypatch):
    _fake_tree(tmp_path, "000000000000")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch("kern_a", "wl") is None


def test_committed_traffic_rows_name_existing_sources():
    """Every row of the committed record names a source file of the library and a 12-digit hash."""
    rows = 0
    for line in open(os.path.join(ROOT, "profiles", "traffic.md")):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 4 and ":" in cells[2] and cells[2].split(":")[0].endswith(".hip"):
            src, digest = cells[2].split(":")
            assert os.path.exists(os.path.join(ROOT, "semi_structured_sparse_sp24_amd", "csrc", src)), src
            assert len(digest) == 12 and int(digest, 16) >= 0
            assert float(cells[3]) > 0
            rows += 1
    assert rows >= 8


def test_layer_audit_needs_every_layer():
    w = inputs.WORKLOADS["prefill"]
    rec = {"eligible": True, "selected": "sparse", "t_sparse_us": 1.0, "t_compress_us": 0.0,
           "t_dense_us": 2.0, "ratio": 2.0, "reason": "", "kernel": "k"}
    full = {(N, K, M): rec for (N, K) in w["shapes"] for M in w["ms"]}
    partial = dict(full)
    partial.pop(next(iter(partial)))
    assert bench.layer_audit("prefill", w, {}, None) is None
    assert bench.layer_audit("prefill", w, partial, None) is None


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
