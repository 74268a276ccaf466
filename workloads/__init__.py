"""Seeded synthetic inputs for the LongFlow decode step.

This package holds workload shapes and random-number recipes only. It computes
no attention, no score and no eviction: the float64 oracle and the HIP path both
take their inputs from here and nothing else is shared between them.
"""
from .configs import WORKLOADS, Workload, get_workload
from .generate import (
    round_to_bf16,
    budgets,
    prefill_lengths,
    prefill_inputs,
    initial_sequence,
    initial_cache,
    step_inputs,
    anchor_positions,
    anchor_event,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "get_workload",
    "round_to_bf16",
    "budgets",
    "prefill_lengths",
    "prefill_inputs",
    "initial_sequence",
    "initial_cache",
    "step_inputs",
    "anchor_positions",
    "anchor_event",
]
