"""Seeded input generators: shapes, reproducibility, bf16 rounding and the
structure each workload promises (anchors, outliers, ragged compressed layout)."""
from __future__ import annotations

import numpy as np
import torch

from workloads import (
    WORKLOADS,
    anchor_event,
    anchor_positions,
    budgets,
    get_workload,
    initial_sequence,
    prefill_lengths,
    round_to_bf16,
    step_inputs,
)
from workloads.generate import outlier_channels


def test_round_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * s for s in (1e-3, 1.0, 1e3)])
    x = np.concatenate([x, np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 0.0], np.float32)])
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_shapes_and_reproducibility():
    for name, w in WORKLOADS.items():
        seqs = [0, w.batch - 1]
        q, k, v = step_inputs(w, 3, seqs)
        assert q.shape == (2, w.n_q_heads, w.head_dim)
        assert k.shape == v.shape == (2, w.n_kv_heads, w.head_dim)
        q2, k2, v2 = step_inputs(w, 3, [w.batch - 1])
        assert np.array_equal(q[1], q2[0]) and np.array_equal(k[1], k2[0]) and np.array_equal(v[1], v2[0])
        if w.dtype == "bf16":
            assert np.array_equal(round_to_bf16(q), q)
        assert not np.array_equal(step_inputs(w, 4, seqs)[0], q)


def test_full_prefill_layout():
    w = get_workload("tiny_f32")
    k, v, pos, t = initial_sequence(w, 0)
    assert k.shape == (2, 256, 64) and t == 256 and np.array_equal(pos, np.arange(256))
    assert abs(k.std() - 1.0) < 0.05


def test_ragged_budgets_and_compressed_layout():
    w = get_workload("ragged_b128")
    bud = budgets(w)
    pre = prefill_lengths(w)
    assert bud.min() >= 1024 and bud.max() <= 8192 and len(set(bud.tolist())) > 100
    assert (pre >= bud).all() and (pre <= 2 * bud).all()
    small = get_workload("ragged_b128").with_(n_kv_heads=1, n_q_heads=5)
    for b in (0, 1, 2):
        k, v, pos, t = initial_sequence(small, b)
        assert k.shape[1] == bud[b] and t == pre[b]
        assert np.array_equal(pos[: w.sink], np.arange(w.sink))
        assert np.array_equal(pos[-w.recent:], np.arange(t - w.recent, t))
        assert (np.diff(pos) > 0).all()


def test_anchor_workload_structure():
    w = get_workload("evict_stress").with_(batch=2)
    ch = outlier_channels(w)
    assert ch.size == 4
    k, v, pos, t = initial_sequence(w, 1)
    ap = anchor_positions(w, 1024)
    assert ap.min() >= w.sink and ap.max() < 1024 - w.recent
    others = np.setdiff1d(np.arange(1024), ap)
    normal_ch = np.setdiff1d(np.arange(128), ch)
    # anchor keys are 2 z with z ~ N(0, I): twice the spread of ordinary keys
    assert k[:, ap][..., normal_ch].std() > 1.6 * k[:, others][..., normal_ch].std()
    # outlier channels carry ten times the spread
    assert k[:, others][..., ch].std() > 8 * k[:, others][..., normal_ch].std()
    assert anchor_event(w, 500) == 0 and anchor_event(w, 1000) == 1 and anchor_event(w, 499) is None
    q, _, _ = step_inputs(w, 500, [1])
    from workloads.generate import anchor_directions
    z = anchor_directions(w, 1)[:, 0, :]
    qq = q[0].reshape(w.n_kv_heads, w.group, -1)
    cos = (qq * z[:, None]).sum(-1) / np.linalg.norm(qq, axis=-1) / np.linalg.norm(z, axis=-1)[:, None]
    assert cos.min() > 0.8
