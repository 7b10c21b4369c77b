"""Layer-level tactic audit manifest.

"Production 2:4 Structured Sparsity for LLMs", section "Audit Artifacts and
Key Metrics": every run yields a manifest with one entry per layer (eligible,
selected, and a reason for every dense choice) and the model-level counts,
the selection ratio and the Sparse GPU-Time Coverage (time of the layers that
run sparse over the total GPU time).  Step 3 of the same page's playbook adds
the eligibility ratio.  The metrics come from sp24_audit_aggregate in the
library; this module only lays the records out per layer.

The audited model is a Llama-3-8B-like stack: 32 blocks of four projections
(fused q/k/v 6144 x 4096, o 4096 x 4096, fused gate/up 28672 x 4096, down
4096 x 14336, as (N, K) of W), the same four shapes the bf16 workloads time.
"""
from __future__ import annotations

import hashlib

from . import audit_aggregate

LLAMA3_8B_BLOCK = (("self_attn.qkv_proj", 6144, 4096), ("self_attn.o_proj", 4096, 4096),
                   ("mlp.gate_up_proj", 28672, 4096), ("mlp.down_proj", 4096, 14336))
LLAMA3_8B_BLOCKS = 32


def synthetic_revision(recipe: str) -> str:
    """Stand-in for a weights revision: the synthetic weights are a function of their seed recipe."""
    return "synthetic-" + hashlib.sha256(recipe.encode()).hexdigest()[:8]


def block_manifest(records_by_shape: dict, model_revision: str, *, blocks: int = LLAMA3_8B_BLOCKS,
                   block=LLAMA3_8B_BLOCK, other_time_us: float = 0.0, extra: dict | None = None) -> dict:
    """records_by_shape: {(N, K): tactic record dict as select_tactic returns} for every
    projection of `block`; each record stands for that projection in all `blocks` blocks."""
    records = [records_by_shape[(N, K)] for _, N, K in block]
    m = audit_aggregate(records, [blocks] * len(records), other_time_us)
    layers = {}
    for i in range(blocks):
        for (name, _, _), rec in zip(block, records):
            entry = {"eligible": bool(rec["eligible"]), "selected": rec["selected"]}
            if rec["selected"] != "sparse":
                entry["reason"] = rec["reason"]
            layers[f"model.layers.{i}.{name}"] = entry
    manifest = {
        "model_revision": model_revision,
        "sparsity_pattern": "2:4",
        "metrics": {
            "candidate_layers": m["candidate_layers"],
            "eligible_layers": m["eligible_layers"],
            "sparse_selected_layers": m["sparse_selected_layers"],
            "dense_fallback_layers": m["dense_fallback_layers"],
            "eligibility_ratio": round(m["eligibility_ratio"], 4),
            "sparse_selection_ratio": round(m["sparse_selection_ratio"], 4),
            "sparse_gpu_time_coverage": round(m["sparse_gpu_time_coverage"], 4),
            "sparse_gpu_time_us": round(m["sparse_gpu_time_us"], 3),
            "total_gpu_time_us": round(m["total_gpu_time_us"], 3),
        },
        "layers": layers,
    }
    if extra:
        manifest.update(extra)
    return manifest
