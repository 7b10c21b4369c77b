"""Pins of the oracle's layer-level audit metrics ("Production 2:4 Structured
Sparsity for LLMs", section "Audit Artifacts and Key Metrics", and step 3 of
its playbook): the page's example counts and selection ratio, a coverage
worked by hand, and invariants that any correct aggregation keeps."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "audit_manifest_example.json")


def _rec(eligible, selected, ts=0.0, tc=0.0, td=0.0):
    return dict(eligible=eligible, selected=selected, t_sparse_us=ts, t_compress_us=tc, t_dense_us=td)


def test_page_example_counts_and_selection_ratio():
    g = json.load(open(GOLDEN))["metrics"]
    # 96 eligible layers, 71 of them running sparse, as in the page's manifest
    m = oracle.audit_metrics([_rec(True, "sparse", 10.0), _rec(True, "dense", 0.0, 0.0, 9.0)], [71, 25])
    assert m["candidate_layers"] == g["candidate_layers"]
    assert m["eligible_layers"] == g["eligible_layers"]
    assert m["sparse_selected_layers"] == g["sparse_selected_layers"]
    assert m["dense_fallback_layers"] == g["dense_fallback_layers"]
    assert round(m["sparse_selection_ratio"], 4) == g["sparse_selection_ratio"]


def test_coverage_worked_by_hand():
    # 3 sparse layers of 10 + 1 us (an online operand pays its compress), 2 ineligible
    # dense layers of 5 us, 4 us outside the audited layers: 33 / (33 + 10 + 4)
    m = oracle.audit_metrics([_rec(True, "sparse", 10.0, 1.0, 20.0), _rec(False, "dense", 0.0, 0.0, 5.0)],
                             [3, 2], 4.0)
    assert (m["candidate_layers"], m["eligible_layers"], m["sparse_selected_layers"],
            m["dense_fallback_layers"]) == (5, 3, 3, 2)
    assert m["eligibility_ratio"] == 3 / 5
    assert m["sparse_selection_ratio"] == 1.0
    assert m["sparse_gpu_time_us"] == 33.0 and m["total_gpu_time_us"] == 47.0
    assert abs(m["sparse_gpu_time_coverage"] - 33 / 47) < 1e-15


def _random_records(rng, n):
    recs = []
    for _ in range(n):
        el = bool(rng.integers(0, 4))
        recs.append(_rec(el, "sparse" if el and rng.integers(0, 2) else "dense",
                         float(rng.uniform(1, 100)), float(rng.uniform(0, 10) * rng.integers(0, 2)),
                         float(rng.uniform(1, 100))))
    return recs, [int(c) for c in rng.integers(0, 40, n)]


def test_invariants():
    rng = np.random.default_rng(5)
    for _ in range(50):
        recs, counts = _random_records(rng, int(rng.integers(1, 9)))
        m = oracle.audit_metrics(recs, counts, float(rng.uniform(0, 50)))
        assert m["sparse_selected_layers"] + m["dense_fallback_layers"] == m["candidate_layers"] == sum(counts)
        assert m["sparse_selected_layers"] <= m["eligible_layers"] <= m["candidate_layers"]
        assert 0.0 <= m["sparse_gpu_time_coverage"] <= 1.0
        # the same layers listed one by one give the same metrics
        flat = [r for r, c in zip(recs, counts) for _ in range(c)]
        m1 = oracle.audit_metrics(flat, [1] * len(flat), 0.0)
        m0 = oracle.audit_metrics(recs, counts, 0.0)
        for k in m0:
            assert abs(m1[k] - m0[k]) <= 1e-9 * max(1.0, abs(m0[k])), k
        # coverage does not depend on the time unit
        scaled = [dict(r, t_sparse_us=3 * r["t_sparse_us"], t_compress_us=3 * r["t_compress_us"],
                       t_dense_us=3 * r["t_dense_us"]) for r in recs]
        assert abs(oracle.audit_metrics(scaled, counts)["sparse_gpu_time_coverage"]
                   - m0["sparse_gpu_time_coverage"]) < 1e-12


def test_extremes():
    # everything sparse and nothing else on the GPU: coverage 1; nothing sparse: 0
    assert oracle.audit_metrics([_rec(True, "sparse", 7.0)], [4])["sparse_gpu_time_coverage"] == 1.0
    assert oracle.audit_metrics([_rec(True, "dense", 7.0, 0.0, 3.0)], [4])["sparse_gpu_time_coverage"] == 0.0
    # a record marked sparse but not eligible still runs dense
    m = oracle.audit_metrics([_rec(False, "sparse", 1.0, 0.0, 2.0)], [3])
    assert m["sparse_selected_layers"] == 0 and m["dense_fallback_layers"] == 3 and m["total_gpu_time_us"] == 6.0
    # no layers at all
    m = oracle.audit_metrics([], [])
    assert m["candidate_layers"] == 0 and m["sparse_gpu_time_coverage"] == 0.0
