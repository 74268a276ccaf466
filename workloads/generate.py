"""Seeded generators for cache contents and per-step inputs.

Every random draw comes from its own PCG64 stream keyed by
``SeedSequence([seed, tag, sequence, step])`` so that any subset of sequences
or steps can be regenerated on its own and gives the same values as the full
batch.  Values are produced as float32 arrays; for bf16 workloads they are
rounded to the nearest bf16 (ties to even) so that the float32 array holds the
exact values stored on the device.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

# Stream tags.
_T_BUDGET = 1
_T_PREFILL = 2
_T_KEEP = 3
_T_CACHE = 4
_T_STEP = 5
_T_OUTLIER = 6
_T_ANCHOR = 7
_T_PREFILL_ROWS = 8


def _rng(w: Workload, tag: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, tag, *ids])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; returns float32.

    Finite inputs only (the generators draw nothing else)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _finish(w: Workload, x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return round_to_bf16(x) if w.dtype == "bf16" else x


def budgets(w: Workload) -> np.ndarray:
    """Per-sequence slot budgets, int32 [batch]."""
    if w.fixed_budget:
        return np.full(w.batch, w.budget_lo, dtype=np.int32)
    r = _rng(w, _T_BUDGET)
    return r.integers(w.budget_lo, w.budget_hi, size=w.batch, endpoint=True).astype(np.int32)


def prefill_lengths(w: Workload) -> np.ndarray:
    """Per-sequence prefill length (tokens seen before the first decode step), int64 [batch]."""
    bud = budgets(w).astype(np.int64)
    if w.prefill == "full":
        return bud.copy()
    if w.prefill == "short":
        return np.minimum(bud, w.prefill_short).astype(np.int64)
    if w.prefill == "ragged":
        r = _rng(w, _T_PREFILL)
        return np.array([r.integers(b, 2 * b, endpoint=True) for b in bud], dtype=np.int64)
    raise ValueError(f"unknown prefill kind {w.prefill!r}")


def outlier_channels(w: Workload) -> np.ndarray:
    """Key channels that carry the outlier scale (same for every head), int64."""
    if w.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(w, _T_OUTLIER)
    return np.sort(r.choice(w.head_dim, size=w.outlier_channels, replace=False)).astype(np.int64)


def anchor_positions(w: Workload, budget: int) -> np.ndarray:
    """Prefill positions of the planted anchors: spread evenly over the middle
    (neither sink nor recent) part of a full prefill of ``budget`` tokens."""
    mid = budget - w.sink - w.recent
    return np.array([w.sink + int((j + 0.5) * mid / w.anchors) for j in range(w.anchors)], dtype=np.int64)


def anchor_directions(w: Workload, b: int) -> np.ndarray:
    """Unit-variance anchor directions z[g][j][:], float64 [Hkv][anchors][d]."""
    r = _rng(w, _T_ANCHOR, b)
    return r.standard_normal((w.n_kv_heads, w.anchors, w.head_dim))


def anchor_event(w: Workload, step: int):
    """Index of the anchor the queries point at on decode step ``step`` (0-based),
    or None.  Events fall on steps anchor_every, 2 anchor_every, ..."""
    if w.anchors == 0 or w.anchor_every <= 0 or step == 0 or step % w.anchor_every:
        return None
    return (step // w.anchor_every - 1) % w.anchors


def _scale_outliers(w: Workload, k: np.ndarray) -> np.ndarray:
    ch = outlier_channels(w)
    if ch.size:
        k[..., ch] *= w.outlier_scale
    return k


def _kept_positions(w: Workload, b: int, budget: int, prefill: int) -> np.ndarray:
    """Positions still cached after the prefill: all of them when the prefill
    fits, else sinks + a seeded sample of the middle + the recent window."""
    if prefill <= budget:
        return np.arange(prefill, dtype=np.int64)
    r = _rng(w, _T_KEEP, b)
    lo, hi = w.sink, prefill - w.recent
    mid = np.sort(r.choice(hi - lo, size=budget - w.sink - w.recent, replace=False)) + lo
    return np.concatenate([np.arange(w.sink), mid, np.arange(hi, prefill)]).astype(np.int64)


def initial_sequence(w: Workload, b: int):
    """Cache contents of sequence ``b`` before the first decode step.

    Returns ``(k, v, pos, t)``: k and v float32 [Hkv][n][d] with the n cached
    tokens in slots 0..n-1 in increasing position order, ``pos`` their
    positions (int64 [n]) and ``t`` the position of the first decoded token."""
    bud = int(budgets(w)[b])
    pre = int(prefill_lengths(w)[b])
    pos = _kept_positions(w, b, bud, pre)
    n = pos.size
    r = _rng(w, _T_CACHE, b)
    k = r.standard_normal((w.n_kv_heads, n, w.head_dim), dtype=np.float32)
    v = r.standard_normal((w.n_kv_heads, n, w.head_dim), dtype=np.float32)
    if w.anchors:
        ap = anchor_positions(w, bud)
        z = anchor_directions(w, b)
        idx = np.searchsorted(pos, ap)
        assert np.array_equal(pos[idx], ap), "anchor positions must be cached"
        k[:, idx, :] = (2.0 * z).astype(np.float32)
    k = _scale_outliers(w, k)
    return _finish(w, k), _finish(w, v), pos, pre


def initial_cache(w: Workload, seqs=None):
    """``initial_sequence`` for several sequences: lists k, v, pos and an int64
    array t, in the order of ``seqs`` (default: all)."""
    seqs = range(w.batch) if seqs is None else seqs
    ks, vs, ps, ts = [], [], [], []
    for b in seqs:
        k, v, p, t = initial_sequence(w, int(b))
        ks.append(k)
        vs.append(v)
        ps.append(p)
        ts.append(t)
    return ks, vs, ps, np.array(ts, dtype=np.int64)


def step_inputs(w: Workload, step: int, seqs=None):
    """Inputs of decode step ``step`` (0-based): q float32 [nb][Hq][d] and
    k_new, v_new float32 [nb][Hkv][d] for the sequences ``seqs`` (default all)."""
    seqs = range(w.batch) if seqs is None else seqs
    ev = anchor_event(w, step)
    qs, ks, vs = [], [], []
    for b in seqs:
        r = _rng(w, _T_STEP, int(b), step)
        q = r.standard_normal((w.n_q_heads, w.head_dim), dtype=np.float32)
        k = r.standard_normal((w.n_kv_heads, w.head_dim), dtype=np.float32)
        v = r.standard_normal((w.n_kv_heads, w.head_dim), dtype=np.float32)
        if ev is not None:
            z = anchor_directions(w, int(b))[:, ev, :]  # [Hkv][d]
            zq = np.repeat(z, w.group, axis=0)  # query head h belongs to kv head h // group
            q = (zq + 0.5 * q.astype(np.float64)).astype(np.float32)
        k = _scale_outliers(w, k)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return _finish(w, np.stack(qs)), _finish(w, np.stack(ks)), _finish(w, np.stack(vs))



def prefill_inputs(w: Workload, max_prefill: int):
    """Full-length prefill of every sequence, for the one-shot compression:
    q_last [B][Hq][d] (the last prefill token's query), k_pre and v_pre
    [B][Hkv][max_prefill][d], N(0,1) draws rounded to the workload's dtype
    (positions past a sequence's prefill length hold draws that are not read)."""
    rng = _rng(w, _T_PREFILL_ROWS)
    q = _finish(w, rng.standard_normal((w.batch, w.n_q_heads, w.head_dim), dtype=np.float32))
    k = _finish(w, rng.standard_normal((w.batch, w.n_kv_heads, max_prefill, w.head_dim), dtype=np.float32))
    v = _finish(w, rng.standard_normal((w.batch, w.n_kv_heads, max_prefill, w.head_dim), dtype=np.float32))
    return q, k, v
