"""GPU parity: the HIP decode step against the float64 oracle, through the C ABI.

Attention outputs within 2e-2 (bf16) / 1e-5 (fp32) absolute, evicted slots
exact outside 1e-6 score ties, importance and log-normaliser checked through
the debug entry point, and the final cache bit-identical to the oracle's."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_harness import log, parity_run
from workloads import budgets, get_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_single_hip_runtime_in_process():
    from kv_cache_eviction_lf_amd import load_library

    load_library()
    torch.zeros(1, device="cuda:0")
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    log(f"libamdhip64 mappings: {paths}")
    assert len(paths) == 1, paths


# ---------------------------------------------------------------- the named workloads

def test_tiny_f32_all_steps_lockstep():
    rep = parity_run(get_workload("tiny_f32"), 512, dbg_every=8)
    assert rep.steps == 512


def test_tiny_f32_free_running():
    # the oracle on its own state; the comparison may only stop at an exempt
    # near-tie (a mismatch anywhere else fails inside the harness)
    rep = parity_run(get_workload("tiny_f32"), 512, free_running=True)
    assert rep.steps == 512 or (rep.diverged_at == rep.steps - 1 and rep.exempt_ties == 1), rep


def test_tiny_f32_vl1_mode():
    rep = parity_run(get_workload("tiny_f32"), 256, score="vl1", dbg_every=8)
    assert rep.steps == 256


def test_llama8b_full_batch_first_steps():
    parity_run(get_workload("llama8b_b8"), 16, dbg_every=4)


def test_llama8b_subset_long_run():
    parity_run(get_workload("llama8b_b8"), 768, check=[0, 7], dbg_every=64)


def test_llama8b_vl1_subset():
    parity_run(get_workload("llama8b_b8"), 64, check=[3], score="vl1", dbg_every=8)


def test_throughput_b64_sampled():
    parity_run(get_workload("throughput_b64"), 48, check=[0, 31, 63], dbg_every=16)


def test_evict_stress_across_anchor_events():
    # crosses the anchor queries of steps 500 and 1000
    parity_run(get_workload("evict_stress"), 1002, check=[0, 1, 2, 15], dbg_every=250)


def test_ragged_b128_sampled():
    w = get_workload("ragged_b128")
    bud = budgets(w)
    check = sorted({0, int(np.argmin(bud)), int(np.argmax(bud))})
    parity_run(w, 40, check=check, dbg_every=13)


# ---------------------------------------------------------------- edge cases

def _small(**kw):
    base = dict(name="edge", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16", budget_lo=300,
                budget_hi=300, sink=4, recent=16, decode_steps=0, seed=11)
    base.update(kw)
    from workloads import Workload

    return Workload(**base)


@pytest.mark.parametrize("kw", [
    dict(prefill="short", prefill_short=100),          # append path, then eviction
    dict(prefill="short", prefill_short=0, budget_lo=40, budget_hi=40, sink=2, recent=4),  # empty cache
    dict(n_q_heads=2, n_kv_heads=2),                   # G = 1
    dict(n_q_heads=16, n_kv_heads=2),                  # G = 8
    dict(n_q_heads=6, n_kv_heads=2, head_dim=64),      # G = 3, d = 64 bf16
    dict(dtype="f32", n_q_heads=10, n_kv_heads=2),     # fp32, d = 128, G = 5
    dict(sink=0, recent=0),                            # no protected window
    dict(budget_lo=21, budget_hi=21, sink=4, recent=16),  # exactly one evictable slot
    dict(budget_lo=200, budget_hi=700, prefill="ragged", batch=5),  # ragged budgets and prefill
])
def test_edge_cases(kw):
    w = _small(**kw)
    steps = 260 if kw.get("prefill") == "short" else 120
    parity_run(w, steps, dbg_every=7, tag=f" {kw}")


@pytest.mark.parametrize("name,steps,check,wait", [
    ("llama8b_b8", 24, None, 0),            # 4 chunks per pair, G = 4: every chunk hands over
    ("evict_stress", 24, [0, 5, 15], 0),    # 4 chunks per pair, G = 7
    ("llama8b_b8", 24, [1, 6], 1),          # a 1 us wait: chunks waiting longer hand over
])
def test_split_chunks_that_do_not_wait(name, steps, check, wait):
    # a split chunk that does not wait for its pair's statistics hands its
    # logits over through memory and the pair's finisher scores them; the
    # results are those of the chunks scoring on chip
    rep = parity_run(get_workload(name), steps, check=check, dbg_every=4, split_wait_us=wait, tag=f" wait={wait}")
    if wait == 0:
        assert rep.deferred == steps * get_workload(name).batch * get_workload(name).n_kv_heads * 4


def test_split_chunks_wait_by_default():
    # the headline shape's 256 work items run at once: no chunk stops waiting
    rep = parity_run(get_workload("llama8b_b8"), 32, check=[0, 7], dbg_every=8)
    assert rep.deferred == 0, rep


def test_small_chunks_and_cache_stride():
    # many chunks with a ragged last one, and a slot stride larger than every budget
    w = _small(budget_lo=333, budget_hi=333, batch=2)
    parity_run(w, 80, chunk_slots=128, max_budget=512, dbg_every=5)


@pytest.mark.parametrize("kw,chunk", [
    (dict(budget_lo=1000, budget_hi=1000, batch=2), 64),                         # 16 chunks, ragged last
    (dict(budget_lo=4096, budget_hi=4096, batch=1, prefill="full"), 64),         # 64 chunks, the most allowed
    (dict(budget_lo=900, budget_hi=900, batch=2, n_q_heads=14, n_kv_heads=2), 64),  # G = 7: 15 chunks
])
@pytest.mark.parametrize("wait", [None, 0])
def test_many_chunks(kw, chunk, wait):
    # up to the most chunks a pair may have; with and without waiting for the
    # pair's statistics (the finisher then scores every deferred chunk)
    w = _small(**kw)
    parity_run(w, 40, chunk_slots=chunk, dbg_every=4, split_wait_us=wait, tag=f" {kw} chunk={chunk} wait={wait}")


@pytest.mark.parametrize("kw", [
    dict(prefill="short", prefill_short=250),                           # appends, fills, then stores nothing
    dict(prefill="short", prefill_short=250, dtype="f32", n_q_heads=10, n_kv_heads=2),  # fp32, G = 5
    dict(budget_lo=200, budget_hi=700, prefill="ragged", batch=5),      # full from the start, split and not
])
def test_full_cache_comparator(kw):
    # attention only (no importance, no eviction): textbook attention over every
    # stored token plus the incoming one; a full cache stays as it is
    w = _small(**kw)
    parity_run(w, 90, score="none", dbg_every=9, tag=f" none {kw}")


@pytest.mark.parametrize("kw,score", [
    (dict(budget_lo=700, budget_hi=700, batch=2), "attn"),
    (dict(budget_lo=700, budget_hi=700, batch=2), "vl1"),
    # outlier key channels and planted anchors: logits jump within a pass, so
    # the probabilities a resident pair keeps are rescaled mid-stream
    (dict(budget_lo=1024, budget_hi=1024, batch=2, n_q_heads=28, n_kv_heads=4, outlier_channels=4,
          outlier_scale=10.0, anchors=8, anchor_every=7), "attn"),
])
def test_resident_pairs(kw, score):
    # one chunk per pair whose wave ranges fit the LDS buffers: the tail reads
    # the stream's probabilities from LDS instead of logits from memory
    w = _small(**kw)
    parity_run(w, 60, score=score, chunk_slots=1024, dbg_every=5, tag=f" resident {score}")


@pytest.mark.parametrize("kw,score,chunk", [
    (dict(budget_lo=3000, budget_hi=3000, batch=2), "attn", 4096),                 # G = 4
    (dict(budget_lo=3000, budget_hi=3000, batch=2), "vl1", 4096),
    (dict(budget_lo=6000, budget_hi=6000, batch=2, n_q_heads=10, n_kv_heads=2), "vl1", 8192),  # G = 5
    (dict(budget_lo=1500, budget_hi=1500, batch=2, n_q_heads=16, n_kv_heads=2), "attn", 2048),  # G = 8
    (dict(budget_lo=2000, budget_hi=2000, batch=2, n_q_heads=28, n_kv_heads=4, outlier_channels=4,
          outlier_scale=10.0, anchors=8, anchor_every=7), "attn", 2048),           # G = 7, large logits
    (dict(budget_lo=3900, budget_hi=8000, batch=4, prefill="ragged", n_q_heads=10, n_kv_heads=2), "attn",
     8192),                                                                        # G = 5, fp32 and half pairs
    (dict(budget_lo=3000, budget_hi=3000, batch=2, n_q_heads=6, n_kv_heads=2, head_dim=64), "vl1", 4096),  # d 64
    (dict(budget_lo=2500, budget_hi=4000, batch=3, n_q_heads=2, n_kv_heads=2, sink=0, recent=0), "attn",
     4096),                                                                        # G = 1, no windows
])
def test_half_resident_pairs(kw, score, chunk):
    # one chunk per pair whose wave ranges are up to twice the LDS buffers: the
    # stream keeps half-precision logits, the tail bounds every importance from
    # them and scores the possible minima exactly from their key rows
    w = _small(**kw)
    parity_run(w, 30, score=score, chunk_slots=chunk, dbg_every=6, tag=f" half {score}")


@pytest.mark.parametrize("kw,chunk", [
    (dict(budget_lo=5000, budget_hi=5000, batch=2), 8192),                     # bf16 G = 4, wave ranges > 2 buffers
    (dict(budget_lo=300, budget_hi=300, batch=2, dtype="f32", n_q_heads=10, n_kv_heads=2), 320),  # fp32 G = 5
])
def test_unsplit_pairs_logits_through_memory(kw, chunk):
    # one chunk per pair whose logits do not stay on chip: the streaming waves
    # write them to the workspace and the same workgroup's tail reads them back
    w = _small(**kw)
    parity_run(w, 40, chunk_slots=chunk, dbg_every=5, tag=f" unsplit-out {kw.get('dtype', 'bf16')}")


def test_half_resident_equal_importances():
    # every cached key the same: all importances tie, more slots are possible
    # minima than the exact pass takes, and the tail scores every slot exactly;
    # the first eligible slot (just past the sink window) must go
    from kv_cache_eviction_lf_amd import LongFlowCache
    from oracle import OracleCache

    B, Hq, Hkv, D, bud, sink, recent = 1, 8, 2, 128, 4000, 4, 16
    gen = torch.Generator().manual_seed(3)
    bf = lambda *shape: torch.randn(*shape, generator=gen).to(torch.bfloat16)  # noqa: E731
    K = bf(D).expand(B, Hkv, bud, D).contiguous()
    V = bf(B, Hkv, bud, D)
    q, kn, vn = bf(B, Hq, D), bf(B, Hkv, D), bf(B, Hkv, D)
    dev = torch.device("cuda:0")
    Kd, Vd = K.to(dev), V.to(dev)
    cache = LongFlowCache(Kd, Vd, Hq, sink, recent, [bud] * B, budgets=[bud] * B, chunk_slots=8192)
    out, ev = cache.step(q.to(dev), kn.to(dev), vn.to(dev))
    torch.cuda.synchronize()
    f64 = lambda x: x.double().numpy()  # noqa: E731
    oc = OracleCache([f64(K[0])], [f64(V[0])], [np.arange(bud)], [bud], [bud], Hq, sink, recent)
    dec = oc.decide(f64(q), f64(kn), f64(vn))
    assert dec.evict.tolist() == [[sink] * Hkv]
    assert ev.cpu().tolist() == [[sink] * Hkv]
    err = float(np.abs(out.float().cpu().numpy() - dec.out).max())
    assert err <= 2e-2, err
    cache.close()


@pytest.mark.parametrize("score", ["attn", "vl1"])
def test_largest_budget(score):
    # the largest budget the protected-slot bitmap allows (65536 slots), one
    # sequence: 64 chunks per pair, the tail's remainder loop over most logits
    w = _small(budget_lo=65536, budget_hi=65536, batch=1, sink=4, recent=64)
    parity_run(w, 6, score=score, dbg_every=3, tag=f" max budget {score}")


def test_vl1_on_ragged_small():
    w = _small(budget_lo=150, budget_hi=400, prefill="ragged", batch=4, n_q_heads=14, n_kv_heads=2)
    parity_run(w, 100, score="vl1", dbg_every=9)


# ---------------------------------------------------------------- determinism and resume

def _run_steps(w, steps, device, state=None, attach=False, K=None, V=None, start=0, split_wait_us=None):
    from kv_cache_eviction_lf_amd import LongFlowCache
    from workloads.device import device_cache, device_step

    if K is None:
        K, V, seq_len, bud = device_cache(w, device)
    else:
        seq_len, bud = None, budgets(w)
    cache = LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent,
                          seq_len if seq_len is not None else [0] * w.batch, budgets=bud,
                          state=state, attach=attach)
    if split_wait_us is not None:
        cache.set_split_wait(split_wait_us)
    outs, evs = [], []
    for s in range(start, start + steps):
        (qd, kd, vd), _ = device_step(w, s, device)
        o, e = cache.step(qd, kd, vd)
        outs.append(o.clone())
        evs.append(e.clone())
    torch.cuda.synchronize()
    return cache, K, V, outs, evs


def test_bitwise_deterministic():
    w = get_workload("llama8b_b8")
    dev = torch.device("cuda:0")
    log("[determinism] llama8b_b8 twice, 40 steps")
    c1, K1, V1, o1, e1 = _run_steps(w, 40, dev)
    c2, K2, V2, o2, e2 = _run_steps(w, 40, dev)
    for a, b in zip(o1, o2):
        assert torch.equal(a, b)
    for a, b in zip(e1, e2):
        assert torch.equal(a, b)
    assert torch.equal(K1, K2) and torch.equal(V1, V2)
    c1.close()
    c2.close()


@pytest.mark.parametrize("name", ["llama8b_b8", "evict_stress"])
def test_split_paths_agree_bitwise(name):
    # chunks scoring their slots on chip and chunks handing their logits to
    # the finisher give the same bits (outputs, evictions, caches)
    w = get_workload(name)
    dev = torch.device("cuda:0")
    log(f"[split paths] {name}: default wait against no wait, 30 steps")
    c1, K1, V1, o1, e1 = _run_steps(w, 30, dev)
    c2, K2, V2, o2, e2 = _run_steps(w, 30, dev, split_wait_us=0)
    assert c2.check_state().deferred > 0
    for a_, b_ in zip(o1, o2):
        assert torch.equal(a_, b_)
    for a_, b_ in zip(e1, e2):
        assert torch.equal(a_, b_)
    assert torch.equal(K1, K2) and torch.equal(V1, V2)
    c1.close()
    c2.close()


def test_resume_from_saved_state():
    w = get_workload("llama8b_b8").with_(batch=4)
    dev = torch.device("cuda:0")
    log("[resume] 20 steps, snapshot, 20 more; restore, attach, 20 more")
    cache, K, V, _, _ = _run_steps(w, 20, dev)
    snap = (K.clone(), V.clone(), cache.state.clone())
    from workloads.device import device_step

    ref_o, ref_e = [], []
    for s in range(20, 40):
        (qd, kd, vd), _ = device_step(w, s, dev)
        o, e = cache.step(qd, kd, vd)
        ref_o.append(o.clone())
        ref_e.append(e.clone())
    cache.close()
    K2, V2, st2 = snap
    c2, _, _, o2, e2 = _run_steps(w, 20, dev, state=st2, attach=True, K=K2, V=V2, start=20)
    for a, b in zip(ref_o, o2):
        assert torch.equal(a, b)
    for a, b in zip(ref_e, e2):
        assert torch.equal(a, b)
    assert torch.equal(K, K2) and torch.equal(V, V2)
    c2.close()
