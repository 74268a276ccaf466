"""LongFlow-style fused decode step (attention + history-free importance +
argmin eviction + in-place overwrite) for AMD MI355X, behind a C ABI.

``_lib`` is the ctypes binding of include/lf.h with the same function names;
``LongFlowCache`` (one layer) and ``LongFlowLayers`` (a model's layers behind one
handle) wrap it for torch device tensors."""
from ._lib import (
    LF_BF16,
    LF_F32,
    LF_INIT_ATTACH,
    LF_SCORE_ATTN,
    LF_SCORE_NONE,
    LF_SCORE_VL1,
    LFError,
    lf_abi_version,
    lf_decode_step,
    lf_decode_step_dbg,
    lf_decode_step_layer,
    lf_decode_step_layer_dbg,
    lf_free,
    lf_init_cache,
    lf_init_layers,
    lf_last_error,
    lf_probe_copy,
    lf_probe_empty,
    lf_prefill_compress,
    lf_prefill_work_bytes,
    lf_probe_read,
    lf_reset_sequences,
    lf_reset_sequences_budget,
    lf_state_bytes,
    lf_state_bytes_layers,
    load_library,
    make_config,
)


def __getattr__(name):
    if name in ("LongFlowCache", "LongFlowLayers", "compress_prefill"):
        from . import cache

        return getattr(cache, name)
    raise AttributeError(name)


__all__ = [
    "LF_BF16",
    "LF_F32",
    "LF_INIT_ATTACH",
    "LF_SCORE_ATTN",
    "LF_SCORE_NONE",
    "LF_SCORE_VL1",
    "LFError",
    "LongFlowCache",
    "LongFlowLayers",
    "compress_prefill",
    "lf_abi_version",
    "lf_decode_step",
    "lf_decode_step_dbg",
    "lf_decode_step_layer",
    "lf_decode_step_layer_dbg",
    "lf_free",
    "lf_init_cache",
    "lf_init_layers",
    "lf_last_error",
    "lf_probe_copy",
    "lf_probe_empty",
    "lf_prefill_compress",
    "lf_prefill_work_bytes",
    "lf_probe_read",
    "lf_reset_sequences",
    "lf_reset_sequences_budget",
    "lf_state_bytes",
    "lf_state_bytes_layers",
    "load_library",
    "make_config",
]
