"""Float64 CPU oracle of the LongFlow decode step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library."""
from .longflow_oracle import (
    SCORE_ATTN,
    SCORE_NONE,
    SCORE_VL1,
    TIE_TOLERANCE,
    OracleCache,
    StepDecision,
    attention_step,
    prefill_keep,
)

__all__ = ["SCORE_ATTN", "SCORE_NONE", "SCORE_VL1", "TIE_TOLERANCE", "OracleCache", "StepDecision", "attention_step",
           "prefill_keep"]
