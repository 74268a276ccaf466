"""GPU parity of the one-shot prefill compression (lf_prefill_compress) with
the oracle's prefill_keep: the importance of every prefill position within
float32 rounding, the kept positions exactly (where the importance at the
selection threshold is closer than 1e-6 to its neighbour, the GPU's choice is
accepted if every position it swapped lies within 1e-6 of the threshold), the
kept K/V rows bit-exactly, and then decode steps from the compressed cache
against the oracle started from the same kept positions."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import OracleCache, prefill_keep
from workloads import Workload, prefill_inputs

pytestmark = pytest.mark.gpu

TIE = 1e-6


def _case(name, B, Hq, Hkv, d, dtype, budgets, prefill, sink, recent, max_prefill, seed):
    w = Workload(name, B, Hq, Hkv, d, dtype, min(budgets), max(budgets), sink, recent, 0, seed=seed)
    return w, list(budgets), list(prefill), max_prefill


CASES = [
    _case("pf_bf16_g4", 3, 8, 2, 128, "bf16", [300, 512, 512], [700, 512, 1000], 4, 16, 1024, 21),
    _case("pf_f32_g5", 2, 10, 2, 128, "f32", [200, 250], [600, 100], 4, 8, 640, 22),
    _case("pf_bf16_g8_d64", 2, 16, 2, 64, "bf16", [128, 128], [4000, 129], 2, 8, 4096, 23),
    _case("pf_bf16_g1_nowin", 1, 4, 4, 128, "bf16", [1000], [3000], 0, 0, 3072, 24),
    # The ragged batch's shape (G 5, d 128, sink 4, recent 64): its smallest and
    # largest budgets with prefills up to twice the budget, so the decode leg
    # starts from the method's own compression at full size (split pairs).
    _case("pf_ragged_shape", 3, 40, 8, 128, "bf16", [1024, 4096, 8192], [2048, 4100, 16384], 4, 64, 16384, 25),
    # The same shape with every prefill short enough for the selection to keep
    # the importances on chip (the ragged batch's longest prefill is 14801).
    _case("pf_ragged_lds", 2, 40, 8, 128, "bf16", [4096, 7168], [8000, 15000], 4, 64, 15360, 26),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_prefill_compress_matches_oracle(case):
    from kv_cache_eviction_lf_amd import LongFlowCache, compress_prefill

    w, bud, pre, max_prefill = case
    print(f"[prefill] {w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} {w.dtype} "
          f"budgets={bud} prefill={pre} sink={w.sink} recent={w.recent}", flush=True)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = prefill_inputs(w, max_prefill)
    qd, kd, vd = (torch.from_numpy(x).to(dev, tdt) for x in (q, k, v))
    max_budget = max(bud)
    kc, vc, kept, imp = compress_prefill(qd, kd, vd, pre, max_budget, w.sink, w.recent, budgets=bud)
    torch.cuda.synchronize()
    kept_h, imp_h = kept.cpu().numpy(), imp.cpu().numpy().astype(np.float64)
    kc_h, vc_h = kc.float().cpu().numpy(), vc.float().cpu().numpy()
    swapped = 0
    for b in range(w.batch):
        P, nb = pre[b], min(pre[b], bud[b])
        want, imp_o = prefill_keep(k[b, :, :P], q[b], bud[b], w.sink, w.recent)
        err = np.abs(imp_h[b, :, :P] - imp_o) / np.maximum(1e-3, imp_o)
        assert float(err.max()) < 1e-4, f"seq {b}: importance differs by {err.max():.2e} (relative)"
        for g in range(w.n_kv_heads):
            got = kept_h[b, g, :nb]
            assert np.all(kept_h[b, g, nb:] == -1)
            assert np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < P
            if not np.array_equal(got, want[g]):
                # near-ties at the threshold only
                mid = imp_o[g, w.sink:P - w.recent]
                thr = np.sort(mid)[::-1][bud[b] - w.sink - w.recent - 1]
                diff = set(got.tolist()) ^ set(want[g].tolist())
                assert all(abs(imp_o[g, p] - thr) < TIE for p in diff), (b, g, sorted(diff)[:8])
                assert set(range(w.sink)) <= set(got.tolist())
                assert set(range(P - w.recent, P)) <= set(got.tolist())
                swapped += 1
            assert np.array_equal(kc_h[b, g, :nb], k[b, g, got]), f"K rows of ({b},{g})"
            assert np.array_equal(vc_h[b, g, :nb], v[b, g, got]), f"V rows of ({b},{g})"
            assert not kc_h[b, g, nb:].any() and not vc_h[b, g, nb:].any()
    print(f"[prefill] ok, {swapped} near-tie swaps", flush=True)

    # Decode from the compressed cache: positions of the kept tokens are known,
    # the next token's position is P.
    cache = LongFlowCache(kc, vc, w.n_q_heads, w.sink, w.recent, pre, budgets=bud)
    oc = OracleCache([kc_h[b][:, : min(pre[b], bud[b])] for b in range(w.batch)],
                     [vc_h[b][:, : min(pre[b], bud[b])] for b in range(w.batch)],
                     [kept_h[b][:, : min(pre[b], bud[b])] for b in range(w.batch)], pre, bud, w.n_q_heads,
                     w.sink, w.recent)
    rng = np.random.default_rng(w.seed + 1000)
    tol = 2e-2 if w.dtype == "bf16" else 1e-5
    for s in range(12):
        qs = rng.standard_normal((w.batch, w.n_q_heads, w.head_dim)).astype(np.float32)
        ks = rng.standard_normal((w.batch, w.n_kv_heads, w.head_dim)).astype(np.float32)
        vs = rng.standard_normal((w.batch, w.n_kv_heads, w.head_dim)).astype(np.float32)
        qt, kt, vt = (torch.from_numpy(x).to(dev, tdt) for x in (qs, ks, vs))
        qs, ks, vs = (x.float().cpu().numpy() for x in (qt, kt, vt))  # the dtype-rounded values both sides see
        out, ev = cache.step(qt, kt, vt)
        dec = oc.decide(qs, ks, vs)
        assert float(np.abs(out.float().cpu().numpy() - dec.out).max()) <= tol
        ev_h = ev.cpu().numpy()
        slots = dec.slot.copy()
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                if ev_h[b, g] != dec.evict[b, g]:
                    assert dec.accepts(b, g, ev_h[b, g]), (s, b, g, int(ev_h[b, g]), int(dec.evict[b, g]))
                    slots[b, g] = ev_h[b, g]
        oc.commit(slots, ks, vs)
    cache.close()


@pytest.mark.parametrize("max_prefill", [4096, 16384], ids=["lds", "global"])
def test_prefill_equal_importances_keep_the_lowest_positions(max_prefill):
    # Every prefill key of a pair equal: every middle position has the same
    # importance, so the selection runs through its position bits and keeps
    # the lowest middle positions (lower position first on equal importance).
    from kv_cache_eviction_lf_amd import compress_prefill

    B, Hq, Hkv, d, sink, recent = 2, 8, 2, 128, 4, 16
    bud, pre = [300, 1000], [3000, max_prefill - 5]
    print(f"[prefill] equal keys: max_prefill={max_prefill} budgets={bud} prefill={pre}", flush=True)
    rng = np.random.default_rng(31)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(dev, torch.bfloat16)
    row = torch.from_numpy(rng.standard_normal((B, Hkv, 1, d)).astype(np.float32)).to(dev, torch.bfloat16)
    k = row.expand(B, Hkv, max_prefill, d).contiguous()
    v = torch.from_numpy(rng.standard_normal((B, Hkv, max_prefill, d)).astype(np.float32)).to(dev, torch.bfloat16)
    kc, vc, kept, imp = compress_prefill(q, k, v, pre, max(bud), sink, recent, budgets=bud)
    torch.cuda.synchronize()
    kept_h, imp_h = kept.cpu().numpy(), imp.cpu().numpy()
    v_h = v.float().cpu().numpy()
    for b in range(B):
        P, nb = pre[b], bud[b]
        want = np.array(list(range(nb - recent)) + list(range(P - recent, P)))
        for g in range(Hkv):
            assert np.all(imp_h[b, g, :P] == imp_h[b, g, 0]), (b, g)
            assert np.array_equal(kept_h[b, g, :nb], want), (b, g, kept_h[b, g, :8], kept_h[b, g, nb - recent - 4:nb])
            assert np.array_equal(vc[b, g, :nb].float().cpu().numpy(), v_h[b, g, want]), (b, g)


def _large_batch_case():
    # More sequences than travel in the kernel arguments: the lengths, budgets
    # and order are uploaded to the device instead.
    B = 130
    bud = [48 + 8 * (i % 5) for i in range(B)]
    pre = [b + (7 * i) % (b + 1) for i, b in enumerate(bud)]
    return _case("pf_large_batch", B, 4, 1, 64, "bf16", bud, pre, 2, 8, max(pre), 27)


@pytest.mark.parametrize("case", [_large_batch_case()], ids=["pf_large_batch"])
def test_prefill_compress_large_batch(case):
    test_prefill_compress_matches_oracle(case)


def test_prefill_compress_in_a_graph():
    # Batches that fit the kernel arguments make only kernel launches: the call
    # can be captured in a HIP graph; every replay (with eager work and
    # synchronisations between them) must reproduce the eager result.
    from kv_cache_eviction_lf_amd import _lib

    w, bud, pre, max_prefill = CASES[0]
    print(f"[prefill] graph capture: {w.name} budgets={bud} prefill={pre}", flush=True)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in prefill_inputs(w, max_prefill))
    max_budget = max(bud)
    cfg = _lib.make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, max_budget, w.sink, w.recent, _lib.LF_BF16)
    wb = _lib.lf_prefill_work_bytes(cfg, max_prefill)
    work = torch.zeros(wb, dtype=torch.uint8, device=dev)
    shape = (w.batch, w.n_kv_heads, max_budget, w.head_dim)
    kc, vc = torch.zeros(shape, dtype=torch.bfloat16, device=dev), torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    kept = torch.full((w.batch, w.n_kv_heads, max_budget), -1, dtype=torch.int32, device=dev)

    def call(stream):
        _lib.lf_prefill_compress(cfg, bud, pre, max_prefill, q.data_ptr(), k.data_ptr(), v.data_ptr(), kc.data_ptr(),
                                 vc.data_ptr(), kept.data_ptr(), work.data_ptr(), wb, stream)

    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = (kc.clone(), vc.clone(), kept.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        call(torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        kc.zero_()
        vc.zero_()
        kept.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp, name in zip((kc, vc, kept), want, ("k_cache", "v_cache", "kept")):
            assert torch.equal(got, exp), f"replay {rep}: {name} differs from the eager call"
