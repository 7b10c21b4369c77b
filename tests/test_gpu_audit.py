"""The layer-level audit manifest end to end on the GPU: tactic records taken
by sp24_select_tactic for the projections of a small block (one of them
ineligible), laid out per layer, with the metrics of sp24_audit_aggregate
checked against the oracle's aggregation of the same records ("Production 2:4
Structured Sparsity for LLMs", section "Audit Artifacts and Key Metrics")."""
import pytest
import torch

import oracle
import semi_structured_sparse_sp24_amd as sp
from semi_structured_sparse_sp24_amd import audit, inputs
from tests._util import say, to_dev

pytestmark = pytest.mark.gpu

BLOCK = (("mlp.up_proj", 2048, 1024), ("mlp.down_proj", 1024, 2048), ("self_attn.o_proj", 256, 96))


def test_manifest_from_measured_tactics():
    M, blocks = 64, 3
    records = {}
    for i, (name, N, K) in enumerate(BLOCK):
        say("audit tactic", name, M, N, K)
        W = to_dev(inputs.to_bits(inputs.normal((N, K), 0.02, 40 + i), oracle.BF16), oracle.BF16)
        X = to_dev(inputs.to_bits(inputs.normal((M, K), 1.0, 50 + i), oracle.BF16), oracle.BF16)
        v, m = sp.prune_compress(W)
        records[(N, K)] = sp.select_tactic(sp.SPARSE_W, v, m, X, sp.decompress(v, m, K), M, N, K, reps=5)
    torch.cuda.synchronize()
    man = audit.block_manifest(records, "rev-test", blocks=blocks, block=BLOCK, other_time_us=25.0)
    recs = [records[(N, K)] for _, N, K in BLOCK]
    want = oracle.audit_metrics(recs, [blocks] * len(recs), 25.0)
    got = man["metrics"]
    for k in ("candidate_layers", "eligible_layers", "sparse_selected_layers", "dense_fallback_layers"):
        assert got[k] == want[k], k
    for k in ("eligibility_ratio", "sparse_selection_ratio", "sparse_gpu_time_coverage"):
        assert got[k] == round(want[k], 4), k
    assert got["candidate_layers"] == 9 and got["eligible_layers"] == 6
    assert len(man["layers"]) == 9
    o = man["layers"]["model.layers.2.self_attn.o_proj"]
    assert o == {"eligible": False, "selected": "dense", "reason": "Alignment failure"}
    for i in range(blocks):
        for name, N, K in BLOCK[:2]:
            e = man["layers"][f"model.layers.{i}.{name}"]
            assert e["eligible"] and e["selected"] == records[(N, K)]["selected"]
            assert ("reason" in e) == (e["selected"] == "dense")
