"""The C ABI library without a GPU: it loads, exports every symbol the headers
declare, and its host-side validation and state sizing behave as documented.
No call here reaches a kernel or the HIP runtime."""
from __future__ import annotations

import ctypes
from ctypes import c_int32, c_size_t, c_void_p
import os
import re
import subprocess

import pytest

from kv_cache_eviction_lf_amd import _lib
from kv_cache_eviction_lf_amd._lib import LF_ERR_ARG, LF_ERR_STATE, LF_ERR_UNSUPPORTED, LFError, make_config
from workloads import WORKLOADS, budgets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="liblf.so not built")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?(lf_[a-z0-9_]+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"lf_init_cache", "lf_decode_step", "lf_free", "lf_state_bytes", "lf_last_error",
            "lf_decode_step_dbg", "lf_probe_copy", "lf_probe_read", "lf_probe_empty"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert names <= exported, names - exported
    lib = _lib.load_library()
    for n in names:
        assert hasattr(lib, n)
    assert set(_lib.PROTOTYPES) == names


def test_abi_version():
    assert _lib.lf_abi_version() == 2


def _cfg(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, max_budget=512, sink=4, recent=16)
    base.update(kw)
    return make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), LF_ERR_ARG),
    (dict(n_kv_heads=0), LF_ERR_ARG),
    (dict(n_q_heads=7), LF_ERR_ARG),
    (dict(n_q_heads=18), LF_ERR_UNSUPPORTED),  # G = 9
    (dict(head_dim=96), LF_ERR_UNSUPPORTED),
    (dict(dtype=5), LF_ERR_UNSUPPORTED),
    (dict(score=3), LF_ERR_ARG),
    (dict(max_budget=0), LF_ERR_ARG),
    (dict(max_budget=70000), LF_ERR_ARG),
    (dict(sink=-1), LF_ERR_ARG),
    (dict(max_budget=20), LF_ERR_ARG),  # budget 20 <= sink + recent
    (dict(chunk_slots=100), LF_ERR_ARG),  # not a multiple of the tile
    (dict(chunk_slots=128, max_budget=65536), LF_ERR_ARG),  # 512 chunks per pair
])
def test_state_bytes_rejects_bad_configs(kw, status):
    with pytest.raises(LFError) as ei:
        _lib.lf_state_bytes(_cfg(**kw))
    assert ei.value.status == status
    assert _lib.lf_last_error()


def test_state_bytes_rejects_bad_budgets():
    with pytest.raises(LFError) as ei:
        _lib.lf_state_bytes(_cfg(), [512, 513])
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError):
        _lib.lf_state_bytes(_cfg(), [20, 100])  # <= sink + recent


def test_state_bytes_of_the_workloads_are_modest():
    for name, w in WORKLOADS.items():
        cfg = make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.budget_hi, w.sink, w.recent,
                          1 if w.dtype == "bf16" else 0)
        nbytes = _lib.lf_state_bytes(cfg, budgets(w))
        kv_bytes = int(budgets(w).sum()) * w.n_kv_heads * w.head_dim * (2 if w.dtype == "bf16" else 4) * 2
        # logits + partials stay a small fraction of the K/V bytes the step streams
        assert nbytes < 0.15 * kv_bytes + (1 << 20), (name, nbytes, kv_bytes)


def test_init_rejects_null_and_misaligned_pointers_before_any_device_call():
    cfg = _cfg()
    nbytes = _lib.lf_state_bytes(cfg)
    with pytest.raises(LFError) as ei:
        _lib.lf_init_cache(cfg, None, [512, 512], 0, 0, 0, nbytes)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:  # state not 256-byte aligned
        _lib.lf_init_cache(cfg, None, [512, 512], 4096, 8192, 4096 + 16, nbytes)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:  # state too small
        _lib.lf_init_cache(cfg, None, [512, 512], 4096, 8192, 1 << 20, nbytes - 1)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:  # negative seq_len
        _lib.lf_init_cache(cfg, None, [-1, 512], 4096, 8192, 1 << 20, nbytes)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:  # unknown flag
        _lib.lf_init_cache(cfg, None, [1, 512], 4096, 8192, 1 << 20, nbytes, flags=4)
    assert ei.value.status == LF_ERR_ARG


def test_step_rejects_bad_handles_without_launching():
    with pytest.raises(LFError) as ei:
        _lib.lf_decode_step(1, 1, 1, 0, 1, 1)
    assert ei.value.status == LF_ERR_ARG
    fake = (ctypes.c_uint64 * 64)()  # zeroed host memory: wrong magic
    with pytest.raises(LFError) as ei:
        _lib.lf_decode_step(1, 1, 1, ctypes.addressof(fake), 1, 1)
    assert ei.value.status == LF_ERR_STATE
    _lib.lf_free(0)  # NULL-safe
    _lib.lf_free(ctypes.addressof(fake))  # wrong magic: ignored


def test_prefill_compress_validates_before_any_device_call():
    cfg = _cfg()
    wb = _lib.lf_prefill_work_bytes(cfg, 1024)
    assert wb >= 4 * 2 * 2 * 1024 + 16
    good = dict(budgets=None, prefill=[1000, 700], max_prefill=1024, q_last=4096, k_pre=8192, v_pre=12288,
                k_cache=16384, v_cache=20480, kept=24576, work=28672, work_bytes=wb)
    bad = [
        dict(prefill=[1025, 700]),        # longer than max_prefill
        dict(prefill=[0, 700]),           # empty prefill
        dict(q_last=0),                   # NULL
        dict(k_cache=16384 + 8),          # misaligned
        dict(work_bytes=wb - 1),          # scratch too small
        dict(budgets=[20, 512]),          # budget <= sink + recent
        dict(max_prefill=0),
    ]
    for change in bad:
        args = dict(good, **change)
        with pytest.raises(LFError) as ei:
            _lib.lf_prefill_compress(cfg, args["budgets"], args["prefill"], args["max_prefill"], args["q_last"],
                                     args["k_pre"], args["v_pre"], args["k_cache"], args["v_cache"], args["kept"],
                                     args["work"], args["work_bytes"])
        assert ei.value.status == LF_ERR_ARG, change


def test_reset_sequences_rejects_bad_handles_and_arguments():
    with pytest.raises(LFError) as ei:
        _lib.lf_reset_sequences(0, [0], [5])
    assert ei.value.status == LF_ERR_ARG
    fake = (ctypes.c_uint64 * 64)()  # wrong magic
    with pytest.raises(LFError) as ei:
        _lib.lf_reset_sequences(ctypes.addressof(fake), [0], [5])
    assert ei.value.status == LF_ERR_STATE
    with pytest.raises(LFError) as ei:
        _lib.lf_reset_sequences_budget(0, [0], [5], [100])
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:
        _lib.lf_reset_sequences_budget(ctypes.addressof(fake), [0], [5], [100])
    assert ei.value.status == LF_ERR_STATE
    with pytest.raises(ValueError):
        _lib.lf_reset_sequences_budget(0, [0, 1], [5, 5], [100])


def test_prefill_noalloc_rejects_batches_beyond_its_scratch():
    # 128 sequences x 8 KV heads x 16384 prefill positions at G = 5 need far
    # more than the static scratch holds: rejected before any device work
    cfg = _cfg(batch=128, n_q_heads=40, n_kv_heads=8, max_budget=8192, recent=64)
    need = _lib.lf_prefill_work_bytes(cfg, 16384)
    assert need > (64 << 20)
    with pytest.raises(LFError) as ei:
        _lib.lf_prefill_compress_noalloc(cfg, [8192] * 128, [16384] * 128, 16384, 16, 16, 16, 16, 16, 16)
    assert ei.value.status == LF_ERR_ARG
    assert "static scratch" in _lib.lf_last_error()


def test_layers_state_bytes_and_init_validation_before_any_device_call():
    cfg = _cfg()
    one = _lib.lf_state_bytes(cfg)
    assert _lib.lf_state_bytes_layers(cfg, None, 3) == 3 * one
    with pytest.raises(LFError) as ei:
        _lib.lf_state_bytes_layers(cfg, None, 0)
    assert ei.value.status == LF_ERR_ARG
    ks, vs = [4096, 8192, 12288], [16384, 20480, 24576]
    with pytest.raises(LFError) as ei:  # room for two layers only
        _lib.lf_init_layers(cfg, None, [512, 512], ks, vs, 1 << 20, 3 * one - 256)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:  # a NULL layer cache
        _lib.lf_init_layers(cfg, None, [512, 512], [4096, 0, 12288], vs, 1 << 20, 3 * one)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(LFError) as ei:  # a misaligned layer cache
        _lib.lf_init_layers(cfg, None, [512, 512], [4096, 8192 + 4, 12288], vs, 1 << 20, 3 * one)
    assert ei.value.status == LF_ERR_ARG
    with pytest.raises(ValueError):
        _lib.lf_init_layers(cfg, None, [512, 512], ks, vs[:2], 1 << 20, 3 * one)


def test_layer_steps_reject_bad_handles_without_launching():
    with pytest.raises(LFError) as ei:
        _lib.lf_decode_step_layer(1, 1, 1, 0, 0, 1, 1)
    assert ei.value.status == LF_ERR_ARG
    fake = (ctypes.c_uint64 * 64)()
    with pytest.raises(LFError) as ei:
        _lib.lf_decode_step_layer_dbg(1, 1, 1, ctypes.addressof(fake), 0, 1, 1)
    assert ei.value.status == LF_ERR_STATE


def test_probe_read_grid_rejects_bad_grids_before_launching():
    # 16-byte aligned stand-in pointers: the argument checks return before any
    # device call, so this runs without a GPU.
    lib = _lib.load_library()
    for grid in (0, -1, lib.lf_probe_read_sink_words() + 1):
        assert lib.lf_probe_read_grid(c_void_p(4096), c_size_t(64), c_int32(grid), c_void_p(4096), None) == LF_ERR_ARG
    assert lib.lf_probe_read_grid(c_void_p(4096), c_size_t(8), c_int32(1), c_void_p(4096), None) == LF_ERR_ARG
