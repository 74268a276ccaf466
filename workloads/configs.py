"""Workload shapes.

The five named workloads are the decode-step configurations used for parity
and measurement:

* ``tiny_f32``      batch 1, 8 q / 2 kv heads, d 64, fp32, budget 256, sink 4,
                    recent 16, prefill 256, 512 decode steps, seed 0.
* ``llama8b_b8``    batch 8, 32 q / 8 kv heads, d 128, bf16, budget 2048, sink 4,
                    recent 64, prefill 2048, 4096 decode steps.
* ``throughput_b64`` batch 64, 32 q / 8 kv heads, d 128, bf16, budget 4096, sink 4,
                    recent 128, prefill 4096, 16384 decode steps.  A budget of
                    4096 against 16384 generated tokens keeps 20 % of the
                    sequence, the ratio the LongFlow summary quotes for its 80 %
                    compression (LongFlow summary, section 4).
* ``evict_stress``  batch 16, 28 q / 4 kv heads, d 128, bf16, budget 1024, sink 4,
                    recent 64, prefill 1024, 8192 decode steps; 4 key channels
                    scaled x10 and 8 planted anchor keys per (sequence, kv head)
                    that later queries point at every 500 steps.
* ``ragged_b128``   batch 128, 40 q / 8 kv heads, d 128, bf16, budgets uniform in
                    [1024, 8192], prefill uniform in [budget, 2 budget] already
                    compressed to the budget, sink 4, recent 64, 2048 steps.

The pages measure on reasoning benchmarks with real models; these seeded
Gaussian workloads stand in for them (no dataset item is used).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16": storage type of q, k, v, cache and output
    budget_lo: int  # per-sequence budget is uniform in [budget_lo, budget_hi]
    budget_hi: int
    sink: int
    recent: int
    decode_steps: int
    seed: int
    # "full": prefill == budget; "ragged": prefill uniform in [budget, 2 budget]
    # compressed to the budget; "short": prefill shorter than the budget
    # (cache not yet full, exercises the append path).
    prefill: str = "full"
    prefill_short: int = 0  # tokens already cached when prefill == "short"
    outlier_channels: int = 0  # key channels scaled by outlier_scale
    outlier_scale: float = 1.0
    anchors: int = 0  # planted anchor keys per (sequence, kv head)
    anchor_every: int = 0  # decode-step period of the anchor queries
    score: str = "attn"  # "attn" (sum of weights) or "vl1" (weights x |v|_1)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def fixed_budget(self) -> bool:
        return self.budget_lo == self.budget_hi

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 8, 2, 64, "f32", 256, 256, 4, 16, 512, seed=0),
    "llama8b_b8": Workload("llama8b_b8", 8, 32, 8, 128, "bf16", 2048, 2048, 4, 64, 4096, seed=1),
    "throughput_b64": Workload("throughput_b64", 64, 32, 8, 128, "bf16", 4096, 4096, 4, 128, 16384, seed=2),
    "evict_stress": Workload(
        "evict_stress", 16, 28, 4, 128, "bf16", 1024, 1024, 4, 64, 8192, seed=3,
        outlier_channels=4, outlier_scale=10.0, anchors=8, anchor_every=500,
    ),
    "ragged_b128": Workload(
        "ragged_b128", 128, 40, 8, 128, "bf16", 1024, 8192, 4, 64, 2048, seed=4, prefill="ragged",
    ),
}

# Names in the order the workloads are usually listed (tiny parity case first).
ORDER = ["tiny_f32", "llama8b_b8", "throughput_b64", "evict_stress", "ragged_b128"]


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {', '.join(ORDER)}") from None
