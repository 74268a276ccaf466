"""Decode steps captured in a HIP graph (the way the benchmark times them)
against the same steps launched one by one: two caches start from the same
tokens, one advances by eager steps, the other by replays of a captured graph
of the same steps; every output, every evicted slot and the final K/V rows
agree bit for bit (the step is deterministic).  Replays alternate with eager
work and synchronisations, and each replay is checked."""
from __future__ import annotations

import pytest
import torch

from kv_cache_eviction_lf_amd import LongFlowCache
from workloads import Workload
from workloads.device import device_cache

pytestmark = pytest.mark.gpu

STEPS = 6   # steps per graph
ROUNDS = 3  # replays


def _workload(**kw):
    base = dict(name="graph", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16", budget_lo=1000,
                budget_hi=1000, sink=4, recent=16, decode_steps=0, seed=41)
    base.update(kw)
    return Workload(**base)


@pytest.mark.parametrize("kw", [
    dict(),                                               # bf16, split pairs (4 pairs, chunks per pair > 1)
    dict(dtype="f32", n_q_heads=10, budget_lo=300, budget_hi=300),  # fp32 vector-ALU path, G = 5
    dict(budget_lo=200, budget_hi=700, prefill="ragged", batch=5),  # ragged budgets: work list path
])
def test_graph_replays_match_eager_steps(kw):
    w = _workload(**kw)
    print(f"[graph] {w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} {w.dtype} "
          f"budgets=[{w.budget_lo},{w.budget_hi}]", flush=True)
    dev = torch.device("cuda:0")
    K, V, seq_len, bud = device_cache(w, dev)
    eager = LongFlowCache(K.clone(), V.clone(), w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud)
    graphed = LongFlowCache(K.clone(), V.clone(), w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud)
    dt = K.dtype
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    ins = [(torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=gen, device=dev).to(dt),
            torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=gen, device=dev).to(dt),
            torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=gen, device=dev).to(dt)) for _ in range(STEPS)]
    outs = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dt, device=dev) for _ in range(STEPS)]
    evs = [torch.empty((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev) for _ in range(STEPS)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for s, (q, kn, vn) in enumerate(ins):
            graphed.step(q, kn, vn, outs[s], evs[s])
    for r in range(ROUNDS):
        want = [eager.step(q, kn, vn) for q, kn, vn in ins]
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(0)
        for e in evs:
            e.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(STEPS):
            assert torch.equal(outs[s], want[s][0]), f"replay {r} step {s}: output differs from the eager step"
            assert torch.equal(evs[s], want[s][1]), f"replay {r} step {s}: evictions {evs[s].tolist()} " \
                                                     f"against {want[s][1].tolist()}"
    assert torch.equal(graphed.k_cache, eager.k_cache) and torch.equal(graphed.v_cache, eager.v_cache)
    eager.close()
    graphed.close()
