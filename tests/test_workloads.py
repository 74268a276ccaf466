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


def test_device_step_pool_matches_the_step_recipe():
    # the benchmark's on-device inputs: shapes, dtype, seeded reproducibility,
    # outlier key channels and anchor queries as in step_inputs (on the CPU here)
    from workloads import anchor_event
    from workloads.device import device_step_pool
    from workloads.generate import anchor_directions

    w = get_workload("evict_stress").with_(batch=4)
    ev_step = w.anchor_every  # first anchor event
    a = device_step_pool(w, 3, "cpu", first_step=ev_step - 1)
    b = device_step_pool(w, 3, "cpu", first_step=ev_step - 1)
    for (q, k, v), (q2, k2, v2) in zip(a, b):
        assert q.shape == (w.batch, w.n_q_heads, w.head_dim) and q.dtype == torch.bfloat16
        assert k.shape == v.shape == (w.batch, w.n_kv_heads, w.head_dim)
        assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    ch = outlier_channels(w)
    k = torch.stack([x[1] for x in a]).float()
    rest = np.setdiff1d(np.arange(w.head_dim), ch)
    assert 6.0 < float(k[..., ch].std()) / float(k[..., rest].std()) < 16.0
    assert anchor_event(w, ev_step) is not None and anchor_event(w, ev_step - 1) is None
    q_ev = a[1][0].double().numpy()
    z = np.stack([anchor_directions(w, s) for s in range(w.batch)])[:, :, anchor_event(w, ev_step), :]
    zq = np.repeat(z, w.group, axis=1)
    resid = q_ev - zq  # 0.5 N(0, 1) plus bf16 rounding
    assert 0.4 < resid.std() < 0.6
    assert abs(float(a[0][0].double().std()) - 1.0) < 0.1  # no anchor on the step before
