"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, rejects bad arguments before any HIP call, and applies the
tactic decision rule to injected timings.  No GPU is touched."""
import ctypes
import os
import re

import pytest

import semi_structured_sparse_sp24_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sp24.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("sp24_prune_compress", "sp24_decompress", "sp24_gemm", "dense_gemm",
                     "sp24_select_tactic", "sp24_tactic_decide", "sp24_status_str", "sp24_audit_aggregate"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sp.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(sp.SIGNATURES) == set(_declared_functions())


def test_version_and_status_strings():
    assert "gfx950" in sp.version()
    for code in range(6):
        s = sp.lib().sp24_status_str(code).decode()
        assert s.startswith(sp.STATUS[code])
    assert sp.meta_words_per_row(100) == 4 and sp.meta_words_per_row(0) == 0


def _pc(dt=sp.BF16, rows=4, K=64, src=16, ld=None, vals=32, meta=48):
    return sp.lib().sp24_prune_compress(dt, rows, K, src, K if ld is None else ld, vals, meta, None)


def test_prune_compress_validation_precedes_hip():
    assert _pc(dt=sp.F32) == 3                    # fp32 is an output dtype only
    assert _pc(dt=7) == 3
    assert _pc(K=6) == 2                          # K % 4
    assert _pc(rows=-1) == 2
    assert _pc(ld=32) == 2                        # ld < K
    assert _pc(src=None) == 1
    assert _pc(meta=None) == 1
    assert _pc(rows=0) == 0 and _pc(K=0) == 0     # empty: no-op, nothing launched


def _gemm(which=sp.SPARSE_W, in_dt=sp.BF16, out_dt=sp.BF16, M=4, N=16, K=128, v=16, m=32, d=48,
          sx=None, sw=None, y=64):
    return sp.lib().sp24_gemm(which, in_dt, out_dt, M, N, K, v, m, d, sx, sw, y, None)


def test_gemm_validation_precedes_hip():
    assert _gemm(which=3) == 2
    assert _gemm(in_dt=sp.F32) == 3
    assert _gemm(in_dt=sp.E4M3, out_dt=sp.F16) == 3
    assert _gemm(K=6) == 2
    assert _gemm(M=-1) == 2
    assert _gemm(v=None) == 1
    assert _gemm(y=None) == 1
    assert _gemm(K=96) == 4                       # not a multiple of the 64-K step: ineligible
    assert _gemm(in_dt=sp.E4M3, K=192) == 4       # fp8 step is 128
    assert _gemm(d=40) == 4                       # misaligned dense operand
    assert _gemm(y=72) == 4
    assert _gemm(sx=66) == 4                      # misaligned scale vector
    assert _gemm(M=0) == 0 and _gemm(N=0) == 0    # empty output: no-op
    assert sp.lib().dense_gemm(sp.BF16, sp.BF16, 4, 16, 100, 16, 32, None, None, 48, None) == 4
    assert sp.lib().dense_gemm(sp.BF16, sp.BF16, 4, 16, 128, None, 32, None, None, 48, None) == 1


def test_decompress_validation_precedes_hip():
    f = sp.lib().sp24_decompress
    assert f(sp.F32, 4, 64, 16, 32, 48, 64, None) == 3
    assert f(sp.BF16, 4, 66, 16, 32, 48, 66, None) == 2
    assert f(sp.BF16, 4, 64, 16, 32, 48, 60, None) == 2
    assert f(sp.BF16, 4, 64, None, 32, 48, 64, None) == 1


def test_select_tactic_validation():
    rec = sp.Tactic()
    f = sp.lib().sp24_select_tactic
    assert f(0, sp.BF16, sp.BF16, 4, 16, 128, 16, 32, 48, 64, None, None, 80, 1, 0, None, ctypes.byref(rec)) == 2
    assert f(0, sp.BF16, sp.BF16, 4, 16, 128, 16, 32, 48, 64, None, None, 80, 1, 5, None, None) == 1
    # the dense path must be runnable: a null dense operand is an error, not a fallback
    assert f(0, sp.BF16, sp.BF16, 4, 16, 128, 16, 32, 48, None, None, None, 80, 1, 5, None,
             ctypes.byref(rec)) == 1


@pytest.mark.parametrize("fused,plain", [("sp24_quantize_prune_compress", "sp24_quantize_e4m3"),
                                         ("sp24_quantize_i8_prune_compress", "sp24_quantize_i8")])
def test_quantize_validation_precedes_hip(fused, plain):
    f, g = getattr(sp.lib(), fused), getattr(sp.lib(), plain)
    ok = dict(dt=sp.BF16, rows=4, K=64, src=16, ld=64, out=32, meta=48, sc=64)

    def q(**kw):
        a = {**ok, **kw}
        return f(a["dt"], a["rows"], a["K"], a["src"], a["ld"], a["out"], a["meta"], a["sc"], None)
    assert q(dt=sp.E4M3) == 3 and q(dt=sp.F32) == 3          # the source is 16-bit
    assert q(rows=-1) == 2 and q(ld=32) == 2 and q(rows=(1 << 24) + 1) == 2
    assert q(rows=0) == 0 and q(K=0) == 0
    assert q(src=None) == 1 and q(meta=None) == 1 and q(sc=None) == 1
    assert q(K=48, ld=48) == 4                                # whole metadata words only
    assert q(ld=68) == 4 and q(src=24) == 4 and q(sc=66) == 4
    assert g(sp.F16, 4, 64, 16, 64, None, 64, None) == 1
    assert g(sp.F16, 4, 48, 16, 48, 32, 64, None) == 4


def test_gemm_kernel_names_follow_the_dispatch():
    bf = __import__("torch").bfloat16
    k = sp.gemm_kernel
    # decode: up to four dense rows are staged through LDS, five to 16 as 16 staged rows,
    # up to 64 go through registers
    assert k(True, sp.SPARSE_W, bf, bf, 1, 4096, 4096) == "sp24_skinny_x4"
    assert k(True, sp.SPARSE_W, bf, bf, 4, 4096, 4096) == "sp24_skinny_x4"
    assert k(True, sp.SPARSE_W, bf, bf, 16, 4096, 4096) == "sp24_skinny_m16"
    assert k(True, sp.SPARSE_W, bf, bf, 64, 4096, 4096) == "sp24_skinny_m64"
    # 17 to 64 rows: 32-row A tiles once there are 160 of them (5120 rows of W and more)
    assert k(True, sp.SPARSE_W, bf, bf, 64, 6144, 4096) == "sp24_skinny_m64_a32"
    assert k(True, sp.SPARSE_W, bf, bf, 32, 5120, 4096) == "sp24_skinny_m32_a32"
    assert k(True, sp.SPARSE_W, bf, bf, 32, 5104, 4096) == "sp24_skinny_m32"
    assert k(False, sp.SPARSE_W, bf, bf, 64, 6144, 4096) == "dense_skinny_m4_a32"
    assert k(False, sp.SPARSE_W, bf, bf, 32, 5120, 4096) == "dense_skinny_m2_a32"
    assert k(False, sp.SPARSE_W, bf, bf, 16, 4096, 4096) == "dense_skinny_m16"
    # beyond 16 rows: the largest LDS-staged tile that still fills the chip
    assert k(True, sp.SPARSE_W, bf, bf, 8192, 4096, 4096) == "sp24_big_256x256"
    # more than one round of 256x256 tiles, the last at most a quarter of the chip: quarter tiles
    assert k(True, sp.SPARSE_W, bf, bf, 4096, 5120, 5120) == "sp24_big_256x256_tail"        # 320 = 256 + 64
    assert k(True, sp.SPARSE_W, bf, bf, 4096, 4352, 4096) == "sp24_big_256x256_tail"        # 272 = 256 + 16
    assert k(True, sp.SPARSE_X, bf, bf, 5120, 4096, 4096) == "sp24_big_256x256_tail"        # A = X: 20 x 16
    # ... at most half of it: half tiles, in the same tail kernel
    assert k(True, sp.SPARSE_W, bf, bf, 2048, 28672, 4096) == "sp24_big_256x256_tail"       # 896 = 3 * 256 + 128
    assert k(True, sp.SPARSE_W, bf, bf, 4093, 5276, 4096) == "sp24_big_256x256_tail"        # 336 = 256 + 80
    # more than half of it: a last round of whole tiles
    assert k(True, sp.SPARSE_W, bf, bf, 4608, 28672, 4096) == "sp24_big_256x256"            # 2016 = 7 * 256 + 224
    assert k(True, sp.SPARSE_W, bf, bf, 2048, 6144, 4096) == "sp24_big_256x256"             # 192: one round
    assert k(False, sp.SPARSE_W, bf, bf, 4096, 5120, 5120) == "dense_big_256x256_tail"
    assert k(False, sp.SPARSE_W, bf, bf, 2048, 28672, 4096) == "dense_big_256x256_tail"
    # 160 tiles of 256x256 (one round) against 320 of 256x128 (two): the big ones
    assert k(True, sp.SPARSE_W, bf, bf, 2048, 5120, 4096) == "sp24_big_256x256"
    assert k(False, sp.SPARSE_W, bf, bf, 2048, 5120, 4096) == "dense_big_256x256"
    assert k(True, sp.SPARSE_W, bf, bf, 2048, 4096, 4096) == "sp24_big_256x128"
    assert k(True, sp.SPARSE_W, bf, bf, 2048, 4096, 4096) == "sp24_big_256x128"
    assert k(True, sp.SPARSE_W, bf, bf, 512, 4096, 4096) == "sp24_big_128x64"        # 128 tiles of 128x128: fewer than 192
    assert k(True, sp.SPARSE_W, bf, bf, 1024, 4096, 4096) == "sp24_big_128x128"
    assert k(True, sp.SPARSE_W, bf, bf, 64, 28672, 4096) == "sp24_big_128x64"
    assert k(False, sp.SPARSE_W, bf, bf, 8192, 4096, 4096) == "dense_big_256x256"
    assert k(False, sp.SPARSE_W, bf, bf, 512, 4096, 4096) == "dense_big_128x64"
    assert k(False, sp.SPARSE_W, bf, bf, 1024, 4096, 4096) == "dense_big_128x128"
    assert k(False, sp.SPARSE_W, bf, bf, 64, 28672, 4096) == "dense_big_128x64"
    # rejected shapes and degenerate ones
    assert k(True, sp.SPARSE_W, bf, bf, 4, 4096, 96) is None
    assert k(False, sp.SPARSE_W, bf, bf, 4, 4096, 100) is None
    assert k(False, sp.SPARSE_W, bf, bf, 4, 4096, 104) == "dense_skinny_m1"
    assert k(True, sp.SPARSE_W, bf, bf, 0, 4096, 128) == "none"
    assert k(True, sp.SPARSE_W, bf, bf, 4, 4096, 0) == "fill_zero"
    assert k(True, 5, bf, bf, 4, 4096, 128) is None


# ------------------------------------------------------------ decision rule

def test_decide_sparse_strictly_faster():
    r = sp.tactic_decide(True, [10.0, 9.0, 11.0], [12.0, 13.0, 12.5])
    assert r["selected"] == "sparse" and r["t_sparse_us"] == 10.0 and r["t_dense_us"] == 12.5
    assert r["ratio"] == pytest.approx(1.25)
    assert r["reason"] == "Sparse kernel 1.25x faster"


def test_decide_dense_faster_reports_margin():
    r = sp.tactic_decide(True, [11.5, 11.5], [10.0, 10.0])
    assert r["selected"] == "dense"
    assert r["reason"] == "Dense kernel 1.15x faster"        # the form of the pages' manifest example


def test_decide_tie_keeps_dense():
    r = sp.tactic_decide(True, [5.0, 6.0, 7.0], [6.0, 6.0, 6.0])
    assert r["selected"] == "dense" and "Tie" in r["reason"]


def test_decide_uses_medians_not_means():
    # one outlier rep must not flip the choice
    r = sp.tactic_decide(True, [8.0, 8.0, 8.0, 8.0, 1000.0], [9.0, 9.0, 9.0, 9.0, 9.0])
    assert r["selected"] == "sparse"


def test_decide_ineligible_is_dense():
    r = sp.tactic_decide(False, [], [3.0])
    assert r["selected"] == "dense" and not r["eligible"]


def test_decide_rejects_missing_timings():
    with pytest.raises(sp.Sp24Error):
        sp.tactic_decide(True, [], [1.0])
    with pytest.raises(sp.Sp24Error):
        sp.tactic_decide(True, [1.0], [])


def _audit_rec(eligible, selected, ts, tc, td):
    return dict(eligible=eligible, selected=selected, t_sparse_us=ts, t_compress_us=tc, t_dense_us=td,
                ratio=1.0, reason="r", kernel="k")


def test_audit_aggregate_matches_the_oracle():
    import numpy as np
    import oracle
    rng = np.random.default_rng(17)
    for trial in range(40):
        n = int(rng.integers(0, 9))
        recs = []
        for _ in range(n):
            el = bool(rng.integers(0, 4))
            recs.append(_audit_rec(el, "sparse" if rng.integers(0, 2) else "dense", float(rng.uniform(0, 200)),
                                   float(rng.uniform(0, 20) * rng.integers(0, 2)), float(rng.uniform(0, 200))))
        counts = [int(c) for c in rng.integers(0, 64, n)]
        other = float(rng.uniform(0, 100) * rng.integers(0, 2))
        got = sp.audit_aggregate(recs, counts, other)
        want = oracle.audit_metrics(recs, counts, other)
        for k in ("candidate_layers", "eligible_layers", "sparse_selected_layers", "dense_fallback_layers"):
            assert got[k] == want[k], (trial, k)
        for k in ("eligibility_ratio", "sparse_selection_ratio", "sparse_gpu_time_us", "total_gpu_time_us",
                  "sparse_gpu_time_coverage"):
            assert abs(got[k] - want[k]) <= 1e-12 * max(1.0, abs(want[k])), (trial, k)


def test_audit_aggregate_validation():
    lib = sp.lib()
    out = sp.AuditMetrics()
    recs = (sp.Tactic * 1)(sp.tactic_record(_audit_rec(True, "sparse", 1.0, 0.0, 2.0)))
    one = (ctypes.c_int64 * 1)(3)
    assert lib.sp24_audit_aggregate(recs, one, 1, 0.0, None) == 1
    assert lib.sp24_audit_aggregate(None, one, 1, 0.0, ctypes.byref(out)) == 1
    assert lib.sp24_audit_aggregate(recs, None, 1, 0.0, ctypes.byref(out)) == 1
    assert lib.sp24_audit_aggregate(None, None, 0, 0.0, ctypes.byref(out)) == 0 and out.candidate_layers == 0
    assert lib.sp24_audit_aggregate(recs, one, -1, 0.0, ctypes.byref(out)) == 2
    assert lib.sp24_audit_aggregate(recs, one, 1, -1.0, ctypes.byref(out)) == 2
    assert lib.sp24_audit_aggregate(recs, one, 1, float("nan"), ctypes.byref(out)) == 2
    neg = (ctypes.c_int64 * 1)(-1)
    assert lib.sp24_audit_aggregate(recs, neg, 1, 0.0, ctypes.byref(out)) == 2
    bad = (sp.Tactic * 1)(sp.tactic_record(_audit_rec(True, "sparse", float("inf"), 0.0, 2.0)))
    assert lib.sp24_audit_aggregate(bad, one, 1, 0.0, ctypes.byref(out)) == 2
    assert lib.sp24_audit_aggregate(recs, one, 1, 0.0, ctypes.byref(out)) == 0
    assert (out.candidate_layers, out.sparse_selected_layers, out.sparse_gpu_time_coverage) == (3, 3, 1.0)


def test_block_manifest_layout():
    from semi_structured_sparse_sp24_amd import audit
    recs = {}
    for i, (_, N, K) in enumerate(audit.LLAMA3_8B_BLOCK):
        recs[(N, K)] = _audit_rec(i != 1, "sparse" if i in (0, 2) else "dense", 10.0, 0.0, 12.0)
    recs[(4096, 4096)]["reason"] = "Alignment failure"
    m = audit.block_manifest(recs, "rev")
    assert m["sparsity_pattern"] == "2:4" and m["model_revision"] == "rev"
    assert len(m["layers"]) == 4 * audit.LLAMA3_8B_BLOCKS == m["metrics"]["candidate_layers"]
    assert m["metrics"]["sparse_selected_layers"] == 64 and m["metrics"]["eligible_layers"] == 96
    assert m["layers"]["model.layers.31.self_attn.o_proj"] == {"eligible": False, "selected": "dense",
                                                              "reason": "Alignment failure"}
    assert m["layers"]["model.layers.0.mlp.gate_up_proj"] == {"eligible": True, "selected": "sparse"}
    assert "reason" in m["layers"]["model.layers.5.mlp.down_proj"]


def test_hybrid_validation_precedes_hip():
    f = sp.lib().sp24_hybrid_gemm
    ok = dict(dt=sp.BF16, out=sp.BF16, M=4, NS=16, ND=8, K=64, v=16, m=32, wd=48, x=64, sx=None, sw=None, y=80)

    def h(**kw):
        a = {**ok, **kw}
        return f(a["dt"], a["out"], a["M"], a["NS"], a["ND"], a["K"], a["v"], a["m"], a["wd"], a["x"], a["sx"],
                 a["sw"], a["y"], None)
    assert h(dt=sp.F32) == 3 and h(dt=sp.E4M3, out=sp.F16) == 3
    assert h(M=-1) == 2 and h(NS=-8) == 2 and h(ND=-1) == 2 and h(K=62) == 2
    assert h(M=0) == 0 and h(NS=0, ND=0) == 0
    assert h(y=None) == 1 and h(x=None) == 1 and h(v=None) == 1 and h(m=None) == 1 and h(wd=None) == 1
    assert h(K=96) == 4 and h(dt=sp.E4M3, K=64) == 4           # whole sparse steps for both regions
    assert h(NS=12) == 4                                       # dense outputs start on a 16-byte boundary
    assert h(x=72) == 4 and h(wd=56) == 4 and h(y=88) == 4 and h(sw=66) == 4
    k = sp.hybrid_kernel
    bf = __import__("torch").bfloat16
    assert k(bf, bf, 4096, 4096, 1024, 4096) == "sp24_hybrid_256x256"
    # 144 tiles of 256x256 (one round) against 288 of 256x128 (two): the big ones
    assert k(bf, bf, 2048, 3584, 512, 4096) == "sp24_hybrid_256x256"
    assert k(bf, bf, 1536, 2048, 1024, 4096) == "sp24_hybrid_256x128"
    assert k(bf, bf, 64, 4096, 512, 4096) == "sp24_hybrid_128x64"
    assert k(bf, bf, 64, 49152, 512, 4096) == "sp24_hybrid_256x64"
    assert k(bf, bf, 512, 512, 256, 4096) == "sp24_hybrid_128x64"
    assert k(bf, bf, 1000, 2048, 768, 4096) == "sp24_hybrid_128x128"
    assert k(bf, bf, 2048, 4096, 2176, 4096) == "sp24_hybrid_256x256_tail"      # 264 = 256 + 8 tiles
    assert k(bf, bf, 0, 16, 8, 64) == "none" and k(bf, bf, 4, 16, 8, 0) == "fill_zero"
    assert k(bf, bf, 4, 12, 8, 64) is None and k(bf, bf, 4, 16, 8, 96) is None


def test_int8_dtype_rules():
    f = sp.lib().sp24_gemm
    # int8 needs whole 128-K steps and an fp32 / bf16 output; dtype codes past int8 are rejected
    assert f(0, sp.I8, sp.BF16, 4, 16, 64, 16, 32, 48, None, None, 80, None) == 4
    assert f(0, sp.I8, sp.F16, 4, 16, 128, 16, 32, 48, None, None, 80, None) == 3
    assert f(0, 5, sp.BF16, 4, 16, 128, 16, 32, 48, None, None, 80, None) == 3
    i8, bf = __import__("torch").int8, __import__("torch").bfloat16
    assert sp.gemm_kernel(True, sp.SPARSE_W, i8, bf, 1, 4096, 4096) == "sp24_skinny_x4"
    assert sp.gemm_kernel(True, sp.SPARSE_W, i8, bf, 4096, 4096, 4096) == "sp24_big_256x256"
    assert sp.gemm_kernel(False, sp.SPARSE_W, i8, bf, 4096, 4096, 4096) == "dense_big_256x256"
    assert sp.gemm_kernel(True, sp.SPARSE_W, i8, bf, 4, 4096, 64) is None
    # prune+compress accepts int8 (any alignment, a general kernel takes the rest)
    assert sp.lib().sp24_prune_compress(sp.I8, 0, 64, None, 64, None, None, None) == 0


def test_ksplit_validation_precedes_hip():
    f = sp.lib().sp24_ksplit_gemm
    ok = dict(dt=sp.BF16, out=sp.BF16, M=4, N=16, KS=256, K=512, v=16, m=32, wd=48, x=64, sx=None, sw=None, y=80)

    def h(**kw):
        a = {**ok, **kw}
        return f(a["dt"], a["out"], a["M"], a["N"], a["KS"], a["K"], a["v"], a["m"], a["wd"], a["x"], a["sx"],
                 a["sw"], a["y"], None)
    assert h(dt=sp.F32) == 3 and h(dt=sp.E4M3, out=sp.F16) == 3 and h(dt=9) == 3
    assert h(M=-1) == 2 and h(N=-1) == 2 and h(KS=-256) == 2 and h(KS=768) == 2 and h(K=510) == 2
    assert h(M=0) == 0 and h(N=0) == 0
    assert h(y=None) == 1 and h(x=None) == 1 and h(v=None) == 1 and h(m=None) == 1 and h(wd=None) == 1
    assert h(KS=0, v=None, m=None) != 1 and h(KS=512, wd=None) != 1      # an empty range needs no pointer
    assert h(K=480) == 4 and h(dt=sp.E4M3, K=448, KS=256) == 4            # whole K steps
    assert h(KS=128) == 4                                                  # the 2:4 range in 256-column blocks
    assert h(x=72) == 4 and h(wd=56) == 4 and h(y=88) == 4 and h(sw=66) == 4 and h(v=24) == 4
    k = sp.ksplit_kernel
    bf = __import__("torch").bfloat16
    assert k(bf, bf, 4096, 4096, 3072, 4096) == "sp24_ksplit_256x256"
    assert k(bf, bf, 2048, 3072, 2048, 4096) == "sp24_ksplit_256x128"
    assert k(bf, bf, 64, 49152, 256, 4096) == "sp24_ksplit_256x64"
    assert k(bf, bf, 16, 4096, 256, 512) == "sp24_ksplit_128x64"
    assert k(bf, bf, 8192, 4352, 3072, 4096) == "sp24_ksplit_256x256_tail"     # 544 = 2 x 256 + 32 tiles
    assert k(bf, bf, 0, 16, 256, 512) == "none" and k(bf, bf, 4, 16, 0, 0) == "fill_zero"
    assert k(bf, bf, 4, 16, 128, 512) is None and k(bf, bf, 4, 16, 768, 512) is None
