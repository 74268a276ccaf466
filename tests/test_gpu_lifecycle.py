"""Continuous batching on one static cache (lf_reset_sequences): after some
decode steps two sequences of the batch are replaced by new requests (their
rows rewritten, their state restarted), and every sequence, replaced or not,
stays in parity with the float64 oracle that restarts the same sequences from
the same contents."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import OracleCache
from workloads import Workload, initial_sequence
from workloads.device import device_cache, device_step

pytestmark = pytest.mark.gpu


def _check_step(s, out, ev, dec, tol):
    err = float(np.abs(out.float().cpu().numpy() - dec.out).max())
    assert err <= tol, f"step {s}: output differs by {err:.3e}"
    ev_h = ev.cpu().numpy()
    slots = dec.slot.copy()
    for b in range(ev_h.shape[0]):
        for g in range(ev_h.shape[1]):
            if ev_h[b, g] != dec.evict[b, g]:
                assert dec.accepts(b, g, ev_h[b, g]), f"step {s} seq {b} kv {g}: GPU {ev_h[b, g]}, oracle {dec.evict[b, g]}"
                slots[b, g] = ev_h[b, g]
    return slots


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reset_sequences_mid_run(dtype):
    from kv_cache_eviction_lf_amd import LongFlowCache

    w = Workload("lifecycle", 4, 8, 2, 128, dtype, 300, 300, 4, 16, 0, seed=31)
    fresh = w.with_(seed=77, prefill="short", prefill_short=120)  # the new requests
    dev = torch.device("cuda:0")
    print(f"[lifecycle] {dtype}", flush=True)
    K, V, seq_len, bud = device_cache(w, dev)
    cache = LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud)
    init = [initial_sequence(w, b) for b in range(w.batch)]
    oc = OracleCache([x[0] for x in init], [x[1] for x in init], [x[2] for x in init], [x[3] for x in init],
                     bud, w.n_q_heads, w.sink, w.recent)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for s in range(15):
        (qd, kd, vd), (q, kn, vn) = device_step(w, s, dev)
        out, ev = cache.step(qd, kd, vd)
        oc.commit(_check_step(s, out, ev, oc.decide(q, kn, vn), tol), kn, vn)

    replaced = [1, 3]
    lens = []
    for b in replaced:
        k, v, pos, t = initial_sequence(fresh, b)
        n = k.shape[1]
        K[b].zero_()
        V[b].zero_()
        K[b, :, :n] = torch.from_numpy(k).to(K.dtype)
        V[b, :, :n] = torch.from_numpy(v).to(V.dtype)
        one = OracleCache([k], [v], [pos], [t], int(bud[b]), w.n_q_heads, w.sink, w.recent)
        oc.k[b], oc.v[b], oc.pos[b], oc.n[b], oc.t[b] = one.k[0], one.v[0], one.pos[0], one.n[0], one.t[0]
        lens.append(t)
    cache.reset(replaced, lens)

    for s in range(15, 45):
        (qd, kd, vd), (q, kn, vn) = device_step(w, s, dev)
        out, ev = cache.step(qd, kd, vd)
        oc.commit(_check_step(s, out, ev, oc.decide(q, kn, vn), tol), kn, vn)
    assert all(oc.n[b] == 120 + 30 for b in replaced)  # appended after the restart
    Kh, Vh = K.float().cpu().numpy(), V.float().cpu().numpy()
    for b in range(w.batch):
        nb = int(bud[b])
        assert np.array_equal(Kh[b, :, :nb], oc.k[b]) and np.array_equal(Vh[b, :, :nb], oc.v[b]), f"cache of {b}"
    cache.close()


def test_reset_sequences_with_new_budgets():
    # new requests with other budgets take two places (one larger, one smaller
    # and not yet full); the work split changes (equal budgets -> ragged ->
    # equal again) while the other sequences carry on
    from kv_cache_eviction_lf_amd import LongFlowCache, LFError

    w = Workload("rebudget", 4, 8, 2, 128, "bf16", 300, 300, 4, 16, 0, seed=41)
    dev = torch.device("cuda:0")
    print("[lifecycle] new budgets", flush=True)
    K, V, seq_len, bud = device_cache(w, dev, max_budget=512)
    bud = [int(x) for x in bud]
    tight = LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud)
    with pytest.raises(LFError):  # its state buffer holds only the initial layout
        tight.reset([1], [500], budgets=[500])
    tight.close()
    cache = LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud, state_capacity=1 << 22)
    init = [initial_sequence(w, b) for b in range(w.batch)]
    oc = OracleCache([x[0] for x in init], [x[1] for x in init], [x[2] for x in init], [x[3] for x in init],
                     bud, w.n_q_heads, w.sink, w.recent)
    s = 0

    def run(n):
        nonlocal s
        for _ in range(n):
            (qd, kd, vd), (q, kn, vn) = device_step(w, s, dev)
            out, ev = cache.step(qd, kd, vd)
            oc.commit(_check_step(s, out, ev, oc.decide(q, kn, vn), 2e-2), kn, vn)
            s += 1

    def replace(seqs, requests):
        lens, news = [], []
        for b, req in zip(seqs, requests):
            k, v, pos, t = initial_sequence(req, b)
            n = k.shape[1]
            nb = int(req.budget_lo)
            K[b].zero_()
            V[b].zero_()
            K[b, :, :n] = torch.from_numpy(k).to(K.dtype)
            V[b, :, :n] = torch.from_numpy(v).to(V.dtype)
            one = OracleCache([k], [v], [pos], [t], nb, w.n_q_heads, w.sink, w.recent)
            oc.k[b], oc.v[b], oc.pos[b], oc.n[b], oc.t[b] = one.k[0], one.v[0], one.pos[0], one.n[0], one.t[0]
            oc.budget[b] = nb
            bud[b] = nb
            lens.append(t)
            news.append(nb)
        cache.reset(seqs, lens, budgets=news)

    run(12)
    replace([1, 3], [w.with_(seed=77, budget_lo=500, budget_hi=500),
                     w.with_(seed=78, budget_lo=120, budget_hi=120, prefill="short", prefill_short=90)])
    run(40)  # sequence 3 fills its 120 slots and starts evicting
    assert oc.n[3] == 120
    replace([1, 3], [w.with_(seed=79), w.with_(seed=80)])  # every budget 300 again
    run(12)
    Kh, Vh = K.float().cpu().numpy(), V.float().cpu().numpy()
    for b in range(w.batch):
        nb = bud[b]
        assert np.array_equal(Kh[b, :, :nb], oc.k[b]) and np.array_equal(Vh[b, :, :nb], oc.v[b]), f"cache of {b}"
    cache.close()
