"""torch-facing wrapper of the C ABI: device tensors in, device tensors out.

torch provides device memory and the current stream; every step of the decode
path runs in the HIP library (liblf.so), which must be built: there is no
fallback."""
from __future__ import annotations

import torch

from . import _lib
from ._lib import LF_BF16, LF_F32, LF_INIT_ATTACH, LF_SCORE_ATTN, LF_SCORE_NONE, LF_SCORE_VL1

_DTYPES = {torch.bfloat16: LF_BF16, torch.float32: LF_F32}
_SCORES = {"attn": LF_SCORE_ATTN, "vl1": LF_SCORE_VL1, "none": LF_SCORE_NONE}


def _stream_handle(device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on {device}")


class _Handle:
    """Calls shared by the single-layer and the multi-layer handle."""

    handle = 0

    def reset(self, seqs, seq_len, budgets=None) -> None:
        """Restart sequences `seqs` in place (their K/V rows already hold the new
        requests' cached tokens) with `seq_len` tokens seen, in every layer of the
        handle; lf_reset_sequences, or lf_reset_sequences_budget when new
        `budgets` are given for them."""
        if not self.handle:
            raise RuntimeError("cache is closed")
        if budgets is None:
            _lib.lf_reset_sequences(self.handle, list(seqs), list(seq_len), _stream_handle(self.device))
            return
        _lib.lf_reset_sequences_budget(self.handle, list(seqs), list(seq_len), list(budgets),
                                       _stream_handle(self.device))
        full = list(self.budgets) if self.budgets is not None else [self.max_budget] * self.B
        for b, nb in zip(seqs, budgets):
            full[int(b)] = int(nb)
        self.budgets = full

    def set_split_wait(self, max_wait_us: int) -> None:
        """How long a chunk of a split pair waits for the pair's statistics
        before handing its logits over through memory (lf_set_split_wait)."""
        if not self.handle:
            raise RuntimeError("cache is closed")
        _lib.lf_set_split_wait(self.handle, int(max_wait_us))

    def check_state(self):
        """Read the state back and check its invariants in every layer
        (lf_check_state); returns the report (deferred chunks since init, pairs)."""
        if not self.handle:
            raise RuntimeError("cache is closed")
        return _lib.lf_check_state(self.handle, _stream_handle(self.device))

    def close(self) -> None:
        if self.handle:
            _lib.lf_free(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LongFlowCache(_Handle):
    """One layer's static KV cache with per-step LongFlow eviction.

    k_cache, v_cache: contiguous device tensors [B][Hkv][max_budget][d] (bf16 or
    fp32), filled as the C ABI's lf_init_cache describes; budgets: per-sequence
    budgets (None = max_budget); seq_len: tokens already seen per sequence.
    state_capacity: bytes to allocate for the state buffer when none is given
    (at least what the budgets need); a larger buffer lets reset() give
    sequences larger budgets later."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, n_q_heads: int, sink: int, recent: int,
                 seq_len, budgets=None, score: str = "attn", softmax_scale: float = 0.0, chunk_slots: int = 0,
                 state: torch.Tensor | None = None, attach: bool = False, state_capacity: int = 0):
        if k_cache.dim() != 4:
            raise ValueError("k_cache must be [B][Hkv][max_budget][d]")
        if k_cache.dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {k_cache.dtype}")
        self.device = k_cache.device
        B, Hkv, S, d = k_cache.shape
        _need(k_cache, "k_cache", (B, Hkv, S, d), k_cache.dtype, self.device)
        _need(v_cache, "v_cache", (B, Hkv, S, d), k_cache.dtype, self.device)
        self.B, self.Hkv, self.max_budget, self.d = B, Hkv, S, d
        self.Hq = int(n_q_heads)
        self.dtype = k_cache.dtype
        self.k_cache, self.v_cache = k_cache, v_cache
        self.budgets = None if budgets is None else [int(x) for x in budgets]
        self.cfg = _lib.make_config(B, self.Hq, Hkv, d, S, sink, recent, _DTYPES[self.dtype], _SCORES[score],
                                    softmax_scale, chunk_slots)
        self.state_bytes = _lib.lf_state_bytes(self.cfg, self.budgets)
        if state is None:
            if attach:
                raise ValueError("attach needs the saved state tensor")
            state = torch.empty(max(self.state_bytes, int(state_capacity)), dtype=torch.uint8, device=self.device)
        elif state.numel() < self.state_bytes or state.device != self.device:
            raise ValueError("state tensor too small or on another device")
        self.state = state
        self.handle = _lib.lf_init_cache(self.cfg, self.budgets, list(seq_len), k_cache.data_ptr(),
                                         v_cache.data_ptr(), state.data_ptr(), state.numel(),
                                         LF_INIT_ATTACH if attach else 0, _stream_handle(self.device))

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, out: torch.Tensor | None = None,
             evict_idx: torch.Tensor | None = None, scores: torch.Tensor | None = None,
             lse: torch.Tensor | None = None):
        """One fused decode step; returns (out [B][Hq][d], evict_idx int32 [B][Hkv])."""
        return _step(self, None, q, k_new, v_new, out, evict_idx, scores, lse)


class LongFlowLayers(_Handle):
    """The static KV caches of a model's layers behind one handle
    (lf_init_layers): every layer shares the batch, heads, windows, budgets and
    positions; steps run per layer, and reset() restarts sequences in every
    layer at once (with new budgets when given).

    k_caches, v_caches: lists of contiguous device tensors [B][Hkv][max_budget][d],
    one per layer, each filled as the C ABI's lf_init_cache describes;
    state_capacity: bytes for the state buffer when none is given (at least
    what the budgets need for every layer); a larger one lets reset() give
    sequences larger budgets later."""

    def __init__(self, k_caches, v_caches, n_q_heads: int, sink: int, recent: int, seq_len, budgets=None,
                 score: str = "attn", softmax_scale: float = 0.0, chunk_slots: int = 0,
                 state: torch.Tensor | None = None, attach: bool = False, state_capacity: int = 0):
        k_caches, v_caches = list(k_caches), list(v_caches)
        if not k_caches or len(k_caches) != len(v_caches):
            raise ValueError("k_caches and v_caches must be non-empty lists of the same length")
        k0 = k_caches[0]
        if k0.dim() != 4 or k0.dtype not in _DTYPES:
            raise ValueError("caches must be [B][Hkv][max_budget][d] bf16 or fp32 tensors")
        self.device = k0.device
        B, Hkv, S, d = k0.shape
        for i, (k, v) in enumerate(zip(k_caches, v_caches)):
            _need(k, f"k_caches[{i}]", (B, Hkv, S, d), k0.dtype, self.device)
            _need(v, f"v_caches[{i}]", (B, Hkv, S, d), k0.dtype, self.device)
        self.n_layers = len(k_caches)
        self.B, self.Hkv, self.max_budget, self.d = B, Hkv, S, d
        self.Hq = int(n_q_heads)
        self.dtype = k0.dtype
        self.k_caches, self.v_caches = k_caches, v_caches
        self.budgets = None if budgets is None else [int(x) for x in budgets]
        self.cfg = _lib.make_config(B, self.Hq, Hkv, d, S, sink, recent, _DTYPES[self.dtype], _SCORES[score],
                                    softmax_scale, chunk_slots)
        self.state_bytes = _lib.lf_state_bytes_layers(self.cfg, self.budgets, self.n_layers)
        if state is None:
            if attach:
                raise ValueError("attach needs the saved state tensor")
            state = torch.empty(max(self.state_bytes, int(state_capacity)), dtype=torch.uint8, device=self.device)
        elif state.numel() < self.state_bytes or state.device != self.device:
            raise ValueError("state tensor too small or on another device")
        self.state = state
        self.handle = _lib.lf_init_layers(self.cfg, self.budgets, list(seq_len), [k.data_ptr() for k in k_caches],
                                          [v.data_ptr() for v in v_caches], state.data_ptr(), state.numel(),
                                          LF_INIT_ATTACH if attach else 0, _stream_handle(self.device))

    def step(self, layer: int, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             out: torch.Tensor | None = None, evict_idx: torch.Tensor | None = None,
             scores: torch.Tensor | None = None, lse: torch.Tensor | None = None):
        """One fused decode step of layer `layer`; returns (out [B][Hq][d], evict_idx int32 [B][Hkv])."""
        return _step(self, int(layer), q, k_new, v_new, out, evict_idx, scores, lse)


def _step(c, layer, q, k_new, v_new, out, evict_idx, scores, lse):
    if not c.handle:
        raise RuntimeError("cache is closed")
    _need(q, "q", (c.B, c.Hq, c.d), c.dtype, c.device)
    _need(k_new, "k_new", (c.B, c.Hkv, c.d), c.dtype, c.device)
    _need(v_new, "v_new", (c.B, c.Hkv, c.d), c.dtype, c.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", (c.B, c.Hq, c.d), c.dtype, c.device)
    if evict_idx is None:
        evict_idx = torch.empty((c.B, c.Hkv), dtype=torch.int32, device=c.device)
    else:
        _need(evict_idx, "evict_idx", (c.B, c.Hkv), torch.int32, c.device)
    stream = _stream_handle(c.device)
    ptrs = (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), c.handle)
    if scores is not None:
        _need(scores, "scores", (c.B, c.Hkv, c.max_budget), torch.float32, c.device)
    if lse is not None:
        _need(lse, "lse", (c.B, c.Hq), torch.float32, c.device)
    sp = 0 if scores is None else scores.data_ptr()
    lp = 0 if lse is None else lse.data_ptr()
    if layer is None:
        if scores is None and lse is None:
            _lib.lf_decode_step(*ptrs, out.data_ptr(), evict_idx.data_ptr(), stream)
        else:
            _lib.lf_decode_step_dbg(*ptrs, out.data_ptr(), evict_idx.data_ptr(), sp, lp, stream)
    elif scores is None and lse is None:
        _lib.lf_decode_step_layer(*ptrs, layer, out.data_ptr(), evict_idx.data_ptr(), stream)
    else:
        _lib.lf_decode_step_layer_dbg(*ptrs, layer, out.data_ptr(), evict_idx.data_ptr(), sp, lp, stream)
    return out, evict_idx


def compress_prefill(q_last: torch.Tensor, k_pre: torch.Tensor, v_pre: torch.Tensor, prefill, max_budget: int,
                     sink: int, recent: int, budgets=None, softmax_scale: float = 0.0):
    """One-shot compression of prefills longer than their budgets (lf_prefill_compress).

    q_last [B][Hq][d]: query of each sequence's last prefill token; k_pre/v_pre
    [B][Hkv][max_prefill][d]: prefill K/V; prefill: per-sequence prefill length.
    Returns (k_cache, v_cache, kept, importance): caches [B][Hkv][max_budget][d]
    holding the kept tokens in position order in slots 0..min(P_b, budget_b)-1
    (zeros after), kept int32 [B][Hkv][max_budget] positions, importance fp32
    [B][Hkv][max_prefill].  Pass seq_len = prefill to LongFlowCache afterwards."""
    B, Hkv, max_prefill, d = k_pre.shape
    dtype, dev = k_pre.dtype, k_pre.device
    _need(v_pre, "v_pre", k_pre.shape, dtype, dev)
    _need(k_pre, "k_pre", k_pre.shape, dtype, dev)
    if q_last.dim() != 3 or q_last.shape[0] != B or q_last.shape[2] != d:
        raise ValueError(f"q_last has shape {tuple(q_last.shape)}, expected [{B}][Hq][{d}]")
    _need(q_last, "q_last", q_last.shape, dtype, dev)
    if dtype not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    cfg = _lib.make_config(B, q_last.shape[1], Hkv, d, max_budget, sink, recent, _DTYPES[dtype], LF_SCORE_ATTN,
                           softmax_scale, 0)
    wb = _lib.lf_prefill_work_bytes(cfg, max_prefill)
    work = torch.empty(wb, dtype=torch.uint8, device=dev)
    k_cache = torch.zeros((B, Hkv, max_budget, d), dtype=dtype, device=dev)
    v_cache = torch.zeros_like(k_cache)
    kept = torch.full((B, Hkv, max_budget), -1, dtype=torch.int32, device=dev)
    _lib.lf_prefill_compress(cfg, budgets, [int(x) for x in prefill], max_prefill, q_last.data_ptr(),
                             k_pre.data_ptr(), v_pre.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                             kept.data_ptr(), work.data_ptr(), wb, _stream_handle(dev))
    imp = work[: 4 * B * Hkv * max_prefill].view(torch.float32).view(B, Hkv, max_prefill)
    return k_cache, v_cache, kept, imp
