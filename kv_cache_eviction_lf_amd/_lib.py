"""ctypes binding of include/lf.h and include/lf_probe.h.

Argument marshalling only: every function forwards to the C ABI of liblf.so
with the same name and turns a non-zero lf_status into LFError.  Pointers are
plain integers (device addresses, e.g. torch's ``data_ptr()``) and streams are
``hipStream_t`` handles as integers (0 = default stream)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblf.so")

LF_OK, LF_ERR_ARG, LF_ERR_UNSUPPORTED, LF_ERR_STATE, LF_ERR_HIP = range(5)
LF_F32, LF_BF16 = 0, 1
LF_SCORE_ATTN, LF_SCORE_VL1, LF_SCORE_NONE = 0, 1, 2
LF_INIT_ATTACH = 1
STATUS_NAMES = {0: "LF_OK", 1: "LF_ERR_ARG", 2: "LF_ERR_UNSUPPORTED", 3: "LF_ERR_STATE", 4: "LF_ERR_HIP"}


class LFError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class lf_state_report(ctypes.Structure):
    _fields_ = [("deferred", c_uint32), ("n_pairs", c_int32), ("bad_pair", c_int32), ("bad_layer", c_int32)]


class lf_config(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32),
        ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("max_budget", c_int32),
        ("sink", c_int32),
        ("recent", c_int32),
        ("dtype", c_int32),
        ("score", c_int32),
        ("softmax_scale", c_float),
        ("chunk_slots", c_int32),
        ("reserved", c_int32),
    ]


# Exported symbols and their prototypes (restype, argtypes).
PROTOTYPES = {
    "lf_abi_version": (c_int32, []),
    "lf_last_error": (ctypes.c_char_p, []),
    "lf_state_bytes": (c_int32, [POINTER(lf_config), POINTER(c_int32), POINTER(c_size_t)]),
    "lf_init_cache": (
        c_int32,
        [POINTER(lf_config), POINTER(c_int32), POINTER(c_int64), c_void_p, c_void_p, c_void_p, c_size_t, c_int32,
         c_void_p, POINTER(c_void_p)],
    ),
    "lf_state_bytes_layers": (c_int32, [POINTER(lf_config), POINTER(c_int32), c_int32, POINTER(c_size_t)]),
    "lf_init_layers": (
        c_int32,
        [POINTER(lf_config), c_int32, POINTER(c_int32), POINTER(c_int64), POINTER(c_void_p), POINTER(c_void_p),
         c_void_p, c_size_t, c_int32, c_void_p, POINTER(c_void_p)],
    ),
    "lf_decode_step_layer": (
        c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "lf_decode_step_layer_dbg": (
        c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "lf_decode_step": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "lf_decode_step_dbg": (
        c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "lf_free": (None, [c_void_p]),
    "lf_probe_copy": (c_int32, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "lf_probe_read": (c_int32, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "lf_probe_read_sink_words": (c_int32, []),
    "lf_probe_read_grid": (c_int32, [c_void_p, c_size_t, c_int32, c_void_p, c_void_p]),
    "lf_probe_empty": (c_int32, [c_int32, c_void_p]),
    "lf_prefill_work_bytes": (c_int32, [POINTER(lf_config), c_int32, POINTER(c_size_t)]),
    "lf_set_split_wait": (c_int32, [c_void_p, c_int32]),
    "lf_check_state": (c_int32, [c_void_p, c_void_p, POINTER(lf_state_report)]),
    "lf_reset_sequences": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_int64), c_void_p]),
    "lf_reset_sequences_budget": (
        c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_int64), POINTER(c_int32), c_void_p]),
    "lf_prefill_compress": (
        c_int32,
        [POINTER(lf_config), POINTER(c_int32), POINTER(c_int32), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
         c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    ),
    "lf_prefill_compress_noalloc": (
        c_int32,
        [POINTER(lf_config), POINTER(c_int32), POINTER(c_int32), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
         c_void_p, c_void_p, c_void_p],
    ),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblf.so once.  torch is imported first so that the library binds to
    the HIP runtime torch already loaded (same SONAME) and shares its streams."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing; build it with `python -m kv_cache_eviction_lf_amd.build`")
    try:
        import torch  # noqa: F401  (HIP runtime of the process)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != LF_OK:
        msg = load_library().lf_last_error()
        raise LFError(status, func, msg.decode() if msg else "")


def _i32_array(values):
    if values is None:
        return None
    vals = [int(x) for x in values]
    return (c_int32 * len(vals))(*vals)


def make_config(batch, n_q_heads, n_kv_heads, head_dim, max_budget, sink, recent, dtype=LF_BF16,
                score=LF_SCORE_ATTN, softmax_scale=0.0, chunk_slots=0) -> lf_config:
    return lf_config(batch, n_q_heads, n_kv_heads, head_dim, max_budget, sink, recent, dtype, score,
                     softmax_scale, chunk_slots, 0)


def lf_abi_version() -> int:
    return int(load_library().lf_abi_version())


def lf_last_error() -> str:
    msg = load_library().lf_last_error()
    return msg.decode() if msg else ""


def lf_state_bytes(cfg: lf_config, budgets=None) -> int:
    out = c_size_t(0)
    _check(load_library().lf_state_bytes(ctypes.byref(cfg), _i32_array(budgets), ctypes.byref(out)),
           "lf_state_bytes")
    return int(out.value)


def lf_init_cache(cfg: lf_config, budgets, seq_len, k_cache: int, v_cache: int, state: int, state_bytes: int,
                  flags: int = 0, stream: int = 0) -> int:
    sl = [int(x) for x in seq_len]
    sl_arr = (c_int64 * len(sl))(*sl)
    handle = c_void_p(0)
    _check(load_library().lf_init_cache(ctypes.byref(cfg), _i32_array(budgets), sl_arr, c_void_p(k_cache),
                                        c_void_p(v_cache), c_void_p(state), c_size_t(state_bytes), c_int32(flags),
                                        c_void_p(stream), ctypes.byref(handle)), "lf_init_cache")
    return int(handle.value)


def lf_state_bytes_layers(cfg: lf_config, budgets, n_layers: int) -> int:
    out = c_size_t(0)
    _check(load_library().lf_state_bytes_layers(ctypes.byref(cfg), _i32_array(budgets), c_int32(n_layers),
                                                ctypes.byref(out)), "lf_state_bytes_layers")
    return int(out.value)


def lf_init_layers(cfg: lf_config, budgets, seq_len, k_caches, v_caches, state: int, state_bytes: int,
                   flags: int = 0, stream: int = 0) -> int:
    sl = [int(x) for x in seq_len]
    sl_arr = (c_int64 * len(sl))(*sl)
    n = len(k_caches)
    if len(v_caches) != n:
        raise ValueError("k_caches and v_caches must have the same length")
    ks = (c_void_p * max(1, n))(*[c_void_p(int(x)) for x in k_caches])
    vs = (c_void_p * max(1, n))(*[c_void_p(int(x)) for x in v_caches])
    handle = c_void_p(0)
    _check(load_library().lf_init_layers(ctypes.byref(cfg), c_int32(n), _i32_array(budgets), sl_arr, ks, vs,
                                         c_void_p(state), c_size_t(state_bytes), c_int32(flags), c_void_p(stream),
                                         ctypes.byref(handle)), "lf_init_layers")
    return int(handle.value)


def lf_decode_step_layer(q: int, k_new: int, v_new: int, cache: int, layer: int, out: int, evict_idx: int,
                         stream: int = 0) -> None:
    _check(load_library().lf_decode_step_layer(c_void_p(q), c_void_p(k_new), c_void_p(v_new), c_void_p(cache),
                                               c_int32(layer), c_void_p(out), c_void_p(evict_idx), c_void_p(stream)),
           "lf_decode_step_layer")


def lf_decode_step_layer_dbg(q: int, k_new: int, v_new: int, cache: int, layer: int, out: int, evict_idx: int,
                             scores: int = 0, lse: int = 0, stream: int = 0) -> None:
    _check(load_library().lf_decode_step_layer_dbg(c_void_p(q), c_void_p(k_new), c_void_p(v_new), c_void_p(cache),
                                                   c_int32(layer), c_void_p(out), c_void_p(evict_idx),
                                                   c_void_p(scores or None), c_void_p(lse or None),
                                                   c_void_p(stream)), "lf_decode_step_layer_dbg")


def lf_reset_sequences(cache: int, seqs, seq_len, stream: int = 0) -> None:
    s = [int(x) for x in seqs]
    sl = [int(x) for x in seq_len]
    if len(s) != len(sl):
        raise ValueError("seqs and seq_len must have the same length")
    _check(load_library().lf_reset_sequences(c_void_p(cache), c_int32(len(s)), (c_int32 * max(1, len(s)))(*s),
                                             (c_int64 * max(1, len(sl)))(*sl), c_void_p(stream)),
           "lf_reset_sequences")


def lf_reset_sequences_budget(cache: int, seqs, seq_len, budgets, stream: int = 0) -> None:
    s = [int(x) for x in seqs]
    sl = [int(x) for x in seq_len]
    bd = [int(x) for x in budgets]
    if not (len(s) == len(sl) == len(bd)):
        raise ValueError("seqs, seq_len and budgets must have the same length")
    m = max(1, len(s))
    _check(load_library().lf_reset_sequences_budget(c_void_p(cache), c_int32(len(s)), (c_int32 * m)(*s),
                                                    (c_int64 * m)(*sl), (c_int32 * m)(*bd), c_void_p(stream)),
           "lf_reset_sequences_budget")


def lf_prefill_work_bytes(cfg: lf_config, max_prefill: int) -> int:
    out = c_size_t(0)
    _check(load_library().lf_prefill_work_bytes(ctypes.byref(cfg), c_int32(max_prefill), ctypes.byref(out)),
           "lf_prefill_work_bytes")
    return int(out.value)


def lf_prefill_compress(cfg: lf_config, budgets, prefill, max_prefill: int, q_last: int, k_pre: int, v_pre: int,
                        k_cache: int, v_cache: int, kept: int, work: int, work_bytes: int, stream: int = 0) -> None:
    _check(load_library().lf_prefill_compress(
        ctypes.byref(cfg), _i32_array(budgets), _i32_array(prefill), c_int32(max_prefill), c_void_p(q_last),
        c_void_p(k_pre), c_void_p(v_pre), c_void_p(k_cache), c_void_p(v_cache), c_void_p(kept), c_void_p(work),
        c_size_t(work_bytes), c_void_p(stream)), "lf_prefill_compress")


def lf_prefill_compress_noalloc(cfg: lf_config, budgets, prefill, max_prefill: int, q_last: int, k_pre: int,
                                v_pre: int, k_cache: int, v_cache: int, kept: int, stream: int = 0) -> None:
    _check(load_library().lf_prefill_compress_noalloc(
        ctypes.byref(cfg), _i32_array(budgets), _i32_array(prefill), c_int32(max_prefill), c_void_p(q_last),
        c_void_p(k_pre), c_void_p(v_pre), c_void_p(k_cache), c_void_p(v_cache), c_void_p(kept), c_void_p(stream)),
        "lf_prefill_compress_noalloc")


def lf_set_split_wait(cache: int, max_wait_us: int) -> None:
    _check(load_library().lf_set_split_wait(c_void_p(cache), c_int32(max_wait_us)), "lf_set_split_wait")


def lf_check_state(cache: int, stream: int = 0) -> lf_state_report:
    rep = lf_state_report()
    _check(load_library().lf_check_state(c_void_p(cache), c_void_p(stream), ctypes.byref(rep)), "lf_check_state")
    return rep


def lf_decode_step(q: int, k_new: int, v_new: int, cache: int, out: int, evict_idx: int, stream: int = 0) -> None:
    _check(load_library().lf_decode_step(c_void_p(q), c_void_p(k_new), c_void_p(v_new), c_void_p(cache),
                                         c_void_p(out), c_void_p(evict_idx), c_void_p(stream)), "lf_decode_step")


def lf_decode_step_dbg(q: int, k_new: int, v_new: int, cache: int, out: int, evict_idx: int, scores: int = 0,
                       lse: int = 0, stream: int = 0) -> None:
    _check(load_library().lf_decode_step_dbg(c_void_p(q), c_void_p(k_new), c_void_p(v_new), c_void_p(cache),
                                             c_void_p(out), c_void_p(evict_idx), c_void_p(scores or None),
                                             c_void_p(lse or None), c_void_p(stream)), "lf_decode_step_dbg")


def lf_free(cache: int) -> None:
    load_library().lf_free(c_void_p(cache))


def lf_probe_copy(src: int, dst: int, nbytes: int, stream: int = 0) -> None:
    _check(load_library().lf_probe_copy(c_void_p(src), c_void_p(dst), c_size_t(nbytes), c_void_p(stream)),
           "lf_probe_copy")


def lf_probe_read(src: int, nbytes: int, sink: int, stream: int = 0) -> None:
    _check(load_library().lf_probe_read(c_void_p(src), c_size_t(nbytes), c_void_p(sink), c_void_p(stream)),
           "lf_probe_read")


def lf_probe_read_grid(src: int, nbytes: int, n_blocks: int, sink: int, stream: int = 0) -> None:
    _check(load_library().lf_probe_read_grid(c_void_p(src), c_size_t(nbytes), c_int32(n_blocks), c_void_p(sink),
                                             c_void_p(stream)), "lf_probe_read_grid")


def lf_probe_empty(n_blocks: int, stream: int = 0) -> None:
    _check(load_library().lf_probe_empty(c_int32(n_blocks), c_void_p(stream)), "lf_probe_empty")


def lf_probe_read_sink_words() -> int:
    return int(load_library().lf_probe_read_sink_words())
