"""One handle over a model's layer caches (lf_init_layers): every layer steps on
its own inputs through lf_decode_step_layer, and one reset restarts sequences
in every layer, first with the budgets they had, then with new ones.  Each
layer stays in parity with its own float64 oracle cache, and every layer's
cache rows end bit-identical to its oracle's."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import OracleCache
from workloads import Workload, budgets, initial_sequence
from workloads.device import device_cache, device_step

pytestmark = pytest.mark.gpu

N_LAYERS = 3


def _check(layer, s, out, ev, dec, tol):
    err = float(np.abs(out.float().cpu().numpy() - dec.out).max())
    assert err <= tol, f"layer {layer} step {s}: output differs by {err:.3e}"
    ev_h = ev.cpu().numpy()
    slots = dec.slot.copy()
    for b in range(ev_h.shape[0]):
        for g in range(ev_h.shape[1]):
            if ev_h[b, g] != dec.evict[b, g]:
                assert dec.accepts(b, g, ev_h[b, g]), (
                    f"layer {layer} step {s} seq {b} kv {g}: GPU {ev_h[b, g]}, oracle {dec.evict[b, g]}")
                slots[b, g] = ev_h[b, g]
    return slots


def test_layers_step_reset_and_new_budgets():
    from kv_cache_eviction_lf_amd import LFError, LongFlowLayers, _lib

    w = Workload("layers", 4, 8, 2, 128, "bf16", 300, 300, 4, 16, 0, seed=51)
    ws = [w.with_(seed=51 + 1000 * layer) for layer in range(N_LAYERS)]
    dev = torch.device("cuda:0")
    print("[layers] init", flush=True)
    Ks, Vs, ocs = [], [], []
    seq_len, bud = None, None
    for layer in range(N_LAYERS):
        K, V, sl, bd = device_cache(ws[layer], dev, max_budget=512)
        if seq_len is None:
            seq_len, bud = sl, [int(x) for x in bd]
        assert np.array_equal(sl, seq_len)
        Ks.append(K)
        Vs.append(V)
        init = [initial_sequence(ws[layer], b) for b in range(w.batch)]
        ocs.append(OracleCache([x[0] for x in init], [x[1] for x in init], [x[2] for x in init],
                               [x[3] for x in init], bud, w.n_q_heads, w.sink, w.recent))
    cache = LongFlowLayers(Ks, Vs, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud,
                           state_capacity=N_LAYERS << 22)
    s = 0

    def run(n):
        nonlocal s
        for _ in range(n):
            for layer in range(N_LAYERS):  # the layers in turn, as a model's forward pass
                (qd, kd, vd), (q, kn, vn) = device_step(ws[layer], s, dev)
                out, ev = cache.step(layer, qd, kd, vd)
                oc = ocs[layer]
                oc.commit(_check(layer, s, out, ev, oc.decide(q, kn, vn), 2e-2), kn, vn)
            s += 1

    def replace(seqs, make_request, new_budgets):
        lens = None
        for layer in range(N_LAYERS):
            oc, ll = ocs[layer], []
            for b in seqs:
                req = make_request(layer, b)
                k, v, pos, t = initial_sequence(req, b)
                n, nb = k.shape[1], int(budgets(req)[b])
                Ks[layer][b].zero_()
                Vs[layer][b].zero_()
                Ks[layer][b, :, :n] = torch.from_numpy(k).to(Ks[layer].dtype)
                Vs[layer][b, :, :n] = torch.from_numpy(v).to(Vs[layer].dtype)
                one = OracleCache([k], [v], [pos], [t], nb, w.n_q_heads, w.sink, w.recent)
                oc.k[b], oc.v[b], oc.pos[b], oc.n[b], oc.t[b] = one.k[0], one.v[0], one.pos[0], one.n[0], one.t[0]
                oc.budget[b] = nb
                ll.append(t)
            assert lens is None or lens == ll
            lens = ll
        cache.reset(seqs, lens, budgets=new_budgets)
        if new_budgets is not None:
            for b, nb in zip(seqs, new_budgets):
                bud[b] = nb

    run(10)
    print("[layers] reset, same budgets", flush=True)
    replace([2], lambda layer, b: ws[layer].with_(seed=300 + layer), None)
    run(10)
    print("[layers] reset, new budgets", flush=True)
    replace([1, 3], lambda layer, b: (ws[layer].with_(seed=400 + layer, budget_lo=500, budget_hi=500) if b == 1 else
                                      ws[layer].with_(seed=500 + layer, budget_lo=120, budget_hi=120,
                                                      prefill="short", prefill_short=90)), [500, 120])
    run(40)  # sequence 3 fills its 120 slots and starts evicting, in every layer
    assert all(oc.n[3] == 120 for oc in ocs)
    rep = cache.check_state()
    assert rep.bad_layer == -1 and rep.bad_pair == -1
    for layer in range(N_LAYERS):
        Kh, Vh = Ks[layer].float().cpu().numpy(), Vs[layer].float().cpu().numpy()
        oc = ocs[layer]
        for b in range(w.batch):
            nb = bud[b]
            assert np.array_equal(Kh[b, :, :nb], oc.k[b]) and np.array_equal(Vh[b, :, :nb], oc.v[b]), (
                f"layer {layer}: cache of sequence {b}")
    (qd, kd, vd), _ = device_step(ws[0], s, dev)
    with pytest.raises(LFError):  # no such layer: rejected before any launch
        cache.step(N_LAYERS, qd, kd, vd)
    out = torch.empty_like(qd)
    ev = torch.empty((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev)
    with pytest.raises(LFError):  # the single-layer entry point refuses a handle of several layers
        _lib.lf_decode_step(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), cache.handle, out.data_ptr(),
                            ev.data_ptr())
    cache.close()
