"""Pins of the float64 oracle against facts that do not come from the oracle itself:
hand-derived rationals, torch's scaled_dot_product_attention, closed forms,
invariants and a pure-Python brute force."""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import SCORE_ATTN, SCORE_NONE, SCORE_VL1, OracleCache, prefill_keep
from tests.brute import BruteCache
from workloads import get_workload, initial_cache, step_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(s: str) -> float:
    if s.startswith("ln "):
        return math.log(float(Fraction(s[3:])))
    return float(Fraction(s))


# ---------------------------------------------------------------- golden fixture

def _hand_cache(fx, score):
    c = fx["cache"]
    keys = np.array([[math.log(a), math.log(b)] for a, b in zip(c["a"], c["b"])])
    vals = np.array(c["v"], dtype=np.float64)
    return OracleCache([keys[None]], [vals[None]], [c["positions"]], [c["t"]], fx["budget"],
                       fx["n_q_heads"], fx["sink"], fx["recent"], scale=fx["scale"], score=score)


@pytest.mark.parametrize("score", [SCORE_ATTN, SCORE_VL1])
def test_hand_worked_example(score):
    with open(os.path.join(GOLDEN, "hand_worked_step.json")) as f:
        fx = json.load(f)
    oc = _hand_cache(fx, score)
    q = np.array(fx["q"], dtype=np.float64)[None]
    for i, st_ in enumerate(fx["steps"]):
        if score == SCORE_VL1 and "vl1_scores" not in st_:
            break
        kn = np.array([[[math.log(st_["new_a"]), math.log(st_["new_b"])]]])
        vn = np.array([[st_["v_new"]]], dtype=np.float64)
        dec = oc.decide(q, kn, vn)
        want_out = np.array([[_frac(x) for x in row] for row in st_["out"]])
        np.testing.assert_allclose(dec.out[0], want_out, rtol=0, atol=1e-14)
        want_alpha_new = [_frac(row[-1]) for row in st_["alpha"]]
        np.testing.assert_allclose(dec.alpha_new[0], want_alpha_new, rtol=0, atol=1e-15)
        np.testing.assert_allclose(dec.lse[0], [_frac(x) for x in st_["lse"]], rtol=0, atol=1e-14)
        key = "attn" if score == SCORE_ATTN else "vl1"
        np.testing.assert_allclose(dec.scores[0][0], [_frac(x) for x in st_[key + "_scores"]], rtol=0, atol=1e-14)
        assert dec.eligible[0][0].tolist() == st_["eligible"]
        assert int(dec.evict[0, 0]) == st_[key + "_evict"]
        # the tie exemption's measure: second-lowest minus lowest eligible score
        assert abs(float(dec.gap[0, 0]) - _frac(st_[key + "_gap"])) < 1e-14
        oc.commit(dec.slot, kn, vn)
        if "positions_after" in st_:
            assert oc.pos[0][0].tolist() == st_["positions_after"]


# ---------------------------------------------------------------- textbook attention

def _sdpa_reference(keys, vals, q, scale):
    """torch float64 SDPA with GQA: keys/vals [Hkv][n][d], q [Hq][d] -> [Hq][d]."""
    kq = torch.from_numpy(np.asarray(keys, dtype=np.float64))[None]
    vq = torch.from_numpy(np.asarray(vals, dtype=np.float64))[None]
    qq = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 8), (8, 2, 16), (6, 3, 8), (7, 1, 4)])
def test_attention_matches_torch_sdpa_without_eviction(hq, hkv, d):
    rng = np.random.default_rng(10 + hq + d)
    n0, steps, budget = 5, 12, 64
    k0 = rng.standard_normal((hkv, n0, d)).astype(np.float32)
    v0 = rng.standard_normal((hkv, n0, d)).astype(np.float32)
    oc = OracleCache([k0], [v0], [np.arange(n0)], [n0], budget, hq, sink=2, recent=3)
    allk, allv = [k0.astype(np.float64)], [v0.astype(np.float64)]
    for _ in range(steps):
        q = rng.standard_normal((1, hq, d)).astype(np.float32)
        kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        allk.append(kn[0][:, None].astype(np.float64))
        allv.append(vn[0][:, None].astype(np.float64))
        dec = oc.step(q, kn, vn)
        K = np.concatenate(allk, axis=1)
        V = np.concatenate(allv, axis=1)
        ref = _sdpa_reference(K, V, q[0], 1.0 / math.sqrt(d))
        np.testing.assert_allclose(dec.out[0], ref, rtol=0, atol=1e-12)
        assert (dec.evict == -1).all()
        # lse against torch.logsumexp of the per-head logits
        kk = torch.from_numpy(K).repeat_interleave(hq // hkv, dim=0)
        s = torch.einsum("hnd,hd->hn", kk, torch.from_numpy(q[0].astype(np.float64))) / math.sqrt(d)
        np.testing.assert_allclose(dec.lse[0], torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_sdpa_pin_rejects_interleaved_grouping():
    """The GQA pin distinguishes h -> h // G from h -> h % Hkv: feeding the oracle
    queries permuted the interleaved way changes the outputs beyond tolerance."""
    hq, hkv, d = 8, 2, 8
    rng = np.random.default_rng(5)
    k0 = rng.standard_normal((hkv, 6, d)).astype(np.float32)
    v0 = rng.standard_normal((hkv, 6, d)).astype(np.float32)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((1, hkv, d)).astype(np.float32)
    perm = np.array([(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)])
    oc = OracleCache([k0], [v0], [np.arange(6)], [6], 64, hq, 1, 1)
    wrong = oc.decide(q[:, perm], kn, vn).out[0][np.argsort(perm)]
    K = np.concatenate([k0, kn[0][:, None]], axis=1)
    V = np.concatenate([v0, vn[0][:, None]], axis=1)
    ref = _sdpa_reference(K, V, q[0], 1.0 / math.sqrt(d))
    assert np.abs(wrong - ref).max() > 1e-3


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("score", [SCORE_ATTN, SCORE_VL1])
def test_uniform_keys_closed_form(score):
    """Identical keys: every weight is 1/(n+1), the output is the mean of the
    values, ATTN scores are G/(n+1), and the tie goes to the lowest eligible slot."""
    hq, hkv, d, n, sink, recent = 6, 2, 8, 10, 2, 3
    rng = np.random.default_rng(1)
    key = rng.standard_normal(d).astype(np.float32)
    k0 = np.broadcast_to(key, (hkv, n, d)).copy()
    v0 = np.sign(rng.standard_normal((hkv, n, d))).astype(np.float32)  # |v|_1 = d for every slot
    oc = OracleCache([k0], [v0], [np.arange(n)], [n], n, hq, sink, recent, score=score)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    kn = key[None, None].repeat(hkv, 1)
    vn = np.ones((1, hkv, d), np.float32)
    dec = oc.decide(q, kn, vn)
    G = hq // hkv
    for g in range(hkv):
        want = np.concatenate([v0[g], vn[0, g][None]]).astype(np.float64).mean(axis=0)
        for j in range(G):
            np.testing.assert_allclose(dec.out[0, g * G + j], want, rtol=0, atol=1e-14)
        mult = d if score == SCORE_VL1 else 1
        np.testing.assert_allclose(dec.scores[0][g], np.full(n, G * mult / (n + 1)), rtol=1e-14)
        assert dec.evict[0, g] == sink  # all eligible scores tie: lowest eligible slot
        assert dec.gap[0, g] == 0.0  # several slots are correct answers
        assert all(dec.accepts(0, g, e) for e in range(sink, n - recent))
        assert not dec.accepts(0, g, sink - 1) and not dec.accepts(0, g, n - recent)  # protected slots
    np.testing.assert_allclose(dec.alpha_new[0], 1.0 / (n + 1), rtol=1e-14)


def test_weights_of_each_head_sum_to_one():
    w = get_workload("tiny_f32")
    ks, vs, ps, ts = initial_cache(w)
    oc = OracleCache(ks, vs, ps, ts, w.budget_lo, w.n_q_heads, w.sink, w.recent)
    for s in range(3):
        q, kn, vn = step_inputs(w, s)
        dec = oc.step(q, kn, vn)
        G = w.group
        for g in range(w.n_kv_heads):
            total = dec.scores[0][g].sum() + dec.alpha_new[0, g * G:(g + 1) * G].sum()
            assert abs(total - G) < 1e-12


def test_g1_integer_logits_argmin_is_logit_argmin():
    """G = 1, integer-valued q and keys, scale 1: the softmax is monotone in the
    logit, so the evicted slot is the first eligible slot of smallest logit
    (computed here on the exact integer logits)."""
    rng = np.random.default_rng(7)
    d, n, sink, recent = 4, 24, 2, 4
    for trial in range(20):
        k0 = rng.integers(-3, 4, size=(1, n, d)).astype(np.float32)
        q = rng.integers(-2, 3, size=(1, 1, d)).astype(np.float32)
        kn = rng.integers(-3, 4, size=(1, 1, d)).astype(np.float32)
        vn = np.zeros((1, 1, d), np.float32)
        oc = OracleCache([k0], [np.zeros_like(k0)], [np.arange(n)], [n], n, 1, sink, recent, scale=1.0)
        dec = oc.decide(q, kn, vn)
        logits = (k0[0].astype(np.int64) @ q[0, 0].astype(np.int64))
        cand = np.arange(sink, n - recent)
        want = cand[np.argmin(logits[cand])]
        assert dec.evict[0, 0] == want, trial


def test_gap_counts_eligible_slots_only():
    """G = 1, integer logits, scale 1: slot importances are exp(logit) / Z, so
    their order and gaps are fixed by hand.  A protected slot holding the second
    lowest importance does not enter the gap; one eligible slot gives an
    infinite gap; and the acceptance rule takes only the oracle's slot."""
    d, sink, recent = 1, 1, 1
    # slots 0..4 hold positions 0..4; t = 5: slot 0 is the sink, slot 4 the recent window
    logits = np.array([0.0, 1.0, 3.0, 5.0, 2.0])  # eligible slots 1, 2, 3; slot 4 (protected) is 2nd lowest
    k0 = logits.reshape(1, 5, 1).astype(np.float32)
    q = np.ones((1, 1, d), np.float32)
    kn = np.array([[[4.0]]], np.float32)
    oc = OracleCache([k0], [np.zeros_like(k0)], [np.arange(5)], [5], 5, 1, sink, recent, scale=1.0)
    dec = oc.decide(q, kn, np.zeros((1, 1, d), np.float32))
    z = math.exp(0) + math.exp(1) + math.exp(3) + math.exp(5) + math.exp(2) + math.exp(4)
    assert dec.evict[0, 0] == 1
    assert abs(dec.gap[0, 0] - (math.exp(3) - math.exp(1)) / z) < 1e-15  # not exp(2) - exp(1): slot 4 is protected
    assert dec.accepts(0, 0, 1) and not dec.accepts(0, 0, 2) and not dec.accepts(0, 0, 4)
    # a single eligible slot: no second score, infinite gap
    oc1 = OracleCache([k0[:, :3]], [np.zeros_like(k0[:, :3])], [np.arange(3)], [3], 3, 1, sink, recent, scale=1.0)
    dec1 = oc1.decide(q, kn, np.zeros((1, 1, d), np.float32))
    assert dec1.evict[0, 0] == 1 and np.isinf(dec1.gap[0, 0])
    assert not dec1.accepts(0, 0, 0) and not dec1.accepts(0, 0, 2)


def test_accepts_near_ties_only_within_tolerance():
    """Two eligible slots whose importances differ by less than the tolerance:
    both are accepted, a third further away is not, and nothing is accepted in
    place of an append."""
    d = 1
    eps = 1e-9  # logits 1 and 1 + eps give importances about 1e-10 apart
    logits = np.array([0.0, 1.0 + eps, 1.0, 4.0, 0.0])
    k0 = logits.reshape(1, 5, 1)
    q = np.ones((1, 1, d))
    oc = OracleCache([k0], [np.zeros_like(k0)], [np.arange(5)], [5], 5, 1, 1, 1, scale=1.0)
    dec = oc.decide(q, np.array([[[0.0]]]), np.zeros((1, 1, d)))
    assert dec.evict[0, 0] == 2 and dec.gap[0, 0] < 1e-6
    assert dec.accepts(0, 0, 1) and dec.accepts(0, 0, 2) and not dec.accepts(0, 0, 3)
    assert not dec.accepts(0, 0, -1)
    # a cache that is not full appends: only the next free slot is right
    oc2 = OracleCache([k0], [np.zeros_like(k0)], [np.arange(5)], [5], 8, 1, 1, 1, scale=1.0)
    dec2 = oc2.decide(q, np.array([[[0.0]]]), np.zeros((1, 1, d)))
    assert dec2.evict[0, 0] == -1 and dec2.accepts(0, 0, -1) and not dec2.accepts(0, 0, 2)


def test_streaming_closed_form_when_logits_rise_with_position():
    """Constant query and keys whose logit grows with position: the oldest
    eligible token always has the smallest weight, so after every step the cache
    holds the sink positions plus the newest budget - sink positions."""
    d, hq, hkv, budget, sink, recent = 4, 4, 2, 16, 2, 3
    q = np.zeros((1, hq, d), np.float32)
    q[..., 0] = 1.0

    def key(p):
        k = np.zeros(d, np.float32)
        k[0] = 0.25 * p
        return k

    k0 = np.stack([key(p) for p in range(budget)])[None].repeat(hkv, 0)
    v0 = np.ones((hkv, budget, d), np.float32)
    oc = OracleCache([k0], [v0], [np.arange(budget)], [budget], budget, hq, sink, recent, scale=1.0)
    prev_slot = None
    for t in range(budget, budget + 40):
        kn = key(t)[None, None].repeat(hkv, 1)
        dec = oc.step(q, kn, np.ones((1, hkv, d), np.float32))
        want = set(range(sink)) | set(range(t + 1 - (budget - sink), t + 1))
        for g in range(hkv):
            assert set(oc.pos[0][g].tolist()) == want
        # victims cycle through the middle slots in order
        e = int(dec.evict[0, 0])
        if prev_slot is not None:
            assert e == (sink + (prev_slot - sink + 1) % (budget - sink))
        prev_slot = e


def test_vl1_equals_l1_norm_of_removed_contribution():
    """VL1 importance of slot i equals sum over the group's heads of
    |o_h - o_h without token i|_1 at fixed weights (no renormalisation)."""
    rng = np.random.default_rng(3)
    hq, hkv, d, n = 6, 2, 5, 9
    k0 = rng.standard_normal((hkv, n, d)).astype(np.float32)
    v0 = rng.standard_normal((hkv, n, d)).astype(np.float32)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((1, hkv, d)).astype(np.float32)
    oc = OracleCache([k0], [v0], [np.arange(n)], [n], n, hq, 1, 1, score=SCORE_VL1)
    dec = oc.decide(q, kn, vn)
    G = hq // hkv
    scale = 1.0 / math.sqrt(d)
    for g in range(hkv):
        keys = [list(map(float, r)) for r in k0[g]] + [list(map(float, kn[0, g]))]
        vals = [list(map(float, r)) for r in v0[g]] + [list(map(float, vn[0, g]))]
        for i in range(n):
            total = 0.0
            for j in range(G):
                qh = list(map(float, q[0, g * G + j]))
                lg = [scale * sum(a * b for a, b in zip(qh, kk)) for kk in keys]
                m = max(lg)
                w = [math.exp(x - m) for x in lg]
                z = sum(w)
                w = [x / z for x in w]
                full = [sum(w[r] * vals[r][c] for r in range(n + 1)) for c in range(d)]
                minus = [sum(w[r] * vals[r][c] for r in range(n + 1) if r != i) for c in range(d)]
                total += sum(abs(a - b) for a, b in zip(full, minus))
            assert abs(dec.scores[0][g][i] - total) < 1e-12


# ---------------------------------------------------------------- brute force

@settings(max_examples=40, deadline=None)
@given(
    hkv=st.integers(1, 2),
    G=st.sampled_from([1, 2, 3, 4, 7]),
    d=st.sampled_from([2, 4, 8]),
    budget=st.integers(6, 14),
    sink=st.integers(0, 2),
    recent=st.integers(0, 3),
    prefill=st.integers(1, 14),
    vl1=st.booleans(),
    seed=st.integers(0, 10_000),
)
def test_oracle_matches_brute_force(hkv, G, d, budget, sink, recent, prefill, vl1, seed):
    if budget <= sink + recent:
        budget = sink + recent + 1
    prefill = min(prefill, budget)
    rng = np.random.default_rng(seed)
    B, hq = 2, hkv * G
    ks = [rng.standard_normal((hkv, prefill, d)).astype(np.float32) for _ in range(B)]
    vs = [rng.standard_normal((hkv, prefill, d)).astype(np.float32) for _ in range(B)]
    pos = [np.arange(prefill)] * B
    ts = [prefill] * B
    scale = 1.0 / math.sqrt(d)
    oc = OracleCache(ks, vs, pos, ts, budget, hq, sink, recent, score=SCORE_VL1 if vl1 else SCORE_ATTN)
    br = BruteCache(ks, vs, pos, ts, [budget] * B, hq, sink, recent, scale, vl1=vl1)
    for _ in range(2 * budget):
        q = rng.standard_normal((B, hq, d)).astype(np.float32)
        kn = rng.standard_normal((B, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((B, hkv, d)).astype(np.float32)
        dec = oc.decide(q, kn, vn)
        gap_b = br.gaps(q, kn, vn)  # before the step changes the cache
        out_b, slot_b, ev_b = br.step(q, kn, vn)
        np.testing.assert_allclose(dec.out, np.array(out_b), rtol=0, atol=1e-12)
        gb = np.array(gap_b)
        assert (np.isinf(gb) == np.isinf(dec.gap)).all()
        fin = np.isfinite(gb)
        np.testing.assert_allclose(dec.gap[fin], gb[fin], rtol=0, atol=1e-12)
        exact = dec.gap > 1e-12
        assert (np.array(ev_b)[exact] == dec.evict[exact]).all()
        oc.commit(np.array(slot_b), kn, vn)  # follow the brute force inside near-ties
        for b in range(B):
            for g in range(hkv):
                assert oc.pos[b][g, : oc.n[b]].tolist() == br.positions(b, g)


# ---------------------------------------------------------------- invariants over many steps

def test_occupancy_and_protection_over_the_tiny_workload():
    w = get_workload("tiny_f32")
    ks, vs, ps, ts = initial_cache(w)
    oc = OracleCache(ks, vs, ps, ts, w.budget_lo, w.n_q_heads, w.sink, w.recent)
    sink_k = oc.k[0][:, : w.sink].copy()
    for s in range(64):
        q, kn, vn = step_inputs(w, s)
        t = oc.t[0]
        dec = oc.step(q, kn, vn)
        assert oc.n[0] == w.budget_lo
        for g in range(w.n_kv_heads):
            p = oc.pos[0][g]
            assert (p >= 0).all() and len(set(p.tolist())) == w.budget_lo
            e = int(dec.evict[0, g])
            assert w.sink <= e and p[e] == t
            assert set(range(t + 1 - w.recent, t + 1)) <= set(p.tolist())  # recent window kept
            assert np.array_equal(oc.k[0][g, e], kn[0, g])
        assert np.array_equal(oc.k[0][:, : w.sink], sink_k)


def test_append_path_until_full():
    rng = np.random.default_rng(11)
    hkv, hq, d, budget = 2, 4, 4, 8
    k0 = rng.standard_normal((hkv, 3, d)).astype(np.float32)
    oc = OracleCache([k0], [k0.copy()], [np.arange(3)], [3], budget, hq, 1, 2)
    evs = []
    for _ in range(8):
        q = rng.standard_normal((1, hq, d)).astype(np.float32)
        kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        dec = oc.step(q, kn, kn)
        evs.append(int(dec.evict[0, 0]))
    assert evs[:5] == [-1] * 5 and all(e >= 1 for e in evs[5:])
    assert oc.n[0] == budget


def test_rejects_budget_not_above_windows_and_protected_commit():
    k = np.zeros((1, 4, 2), np.float32)
    with pytest.raises(ValueError):
        OracleCache([k], [k], [np.arange(4)], [4], 4, 1, sink=2, recent=2)
    oc = OracleCache([k], [k], [np.arange(4)], [4], 4, 1, sink=1, recent=1)
    with pytest.raises(ValueError):
        oc.commit(np.array([[0]]), np.zeros((1, 1, 2)), np.zeros((1, 1, 2)))


# ---------------------------------------------------------------- full-cache comparator (SCORE_NONE)

@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 16), (7, 1, 4)])
def test_none_mode_is_textbook_attention_then_stops_storing(hq, hkv, d):
    # While there is room every token is kept: SDPA over all of them.  Once the
    # cache is full the token is still attended (SDPA over the stored tokens plus
    # it) but not stored: the cache stays bit-identical and evict is -2.
    rng = np.random.default_rng(40 + hq + d)
    n0, budget, steps = 5, 12, 12
    k0 = rng.standard_normal((hkv, n0, d)).astype(np.float32)
    v0 = rng.standard_normal((hkv, n0, d)).astype(np.float32)
    oc = OracleCache([k0], [v0], [np.arange(n0)], [n0], budget, hq, sink=2, recent=3, score=SCORE_NONE)
    allk, allv = [k0.astype(np.float64)], [v0.astype(np.float64)]
    for step in range(steps):
        q = rng.standard_normal((1, hq, d)).astype(np.float32)
        kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        stored_k = np.concatenate(allk, axis=1)
        stored_v = np.concatenate(allv, axis=1)
        before_k = [x.copy() for x in oc.k]
        dec = oc.step(q, kn, vn)
        K = np.concatenate([stored_k, kn[0][:, None].astype(np.float64)], axis=1)
        V = np.concatenate([stored_v, vn[0][:, None].astype(np.float64)], axis=1)
        np.testing.assert_allclose(dec.out[0], _sdpa_reference(K, V, q[0], 1.0 / math.sqrt(d)), rtol=0, atol=1e-12)
        if n0 + step < budget:
            assert (dec.evict == -1).all() and (dec.slot == n0 + step).all()
            allk.append(kn[0][:, None].astype(np.float64))
            allv.append(vn[0][:, None].astype(np.float64))
        else:
            assert (dec.evict == -2).all()
            assert all(np.array_equal(a, b) for a, b in zip(before_k, oc.k))
        assert oc.n[0] == min(n0 + step + 1, budget)


# ---------------------------------------------------------------- one-shot prefill compression

def _brute_prefill_keep(keys, q, budget, sink, recent):
    """Pure-Python loops: softmax weights with math.exp, importance summed over
    the group's heads, then the middle positions taken one at a time by largest
    importance (first position on equal importance)."""
    Hkv, P, d = len(keys), len(keys[0]), len(keys[0][0])
    G = len(q) // Hkv
    scale = 1.0 / math.sqrt(d)
    out = []
    for g in range(Hkv):
        imp = [0.0] * P
        for j in range(G):
            qh = q[g * G + j]
            s = [scale * sum(qh[x] * keys[g][i][x] for x in range(d)) for i in range(P)]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for i in range(P):
                imp[i] += e[i] / z
        if P <= budget:
            out.append(list(range(P)))
            continue
        left = list(range(sink, P - recent))
        chosen = []
        for _ in range(budget - sink - recent):
            best = left[0]
            for i in left[1:]:
                if imp[i] > imp[best]:
                    best = i
            chosen.append(best)
            left.remove(best)
        out.append(sorted(list(range(sink)) + chosen + list(range(P - recent, P))))
    return out


@pytest.mark.parametrize("seed,Hkv,G,P,budget,sink,recent", [
    (0, 1, 1, 9, 6, 1, 2), (1, 2, 3, 17, 8, 2, 3), (2, 2, 2, 12, 12, 2, 2), (3, 1, 4, 30, 7, 0, 1),
    (4, 3, 1, 25, 10, 3, 0),
])
def test_prefill_keep_matches_brute_force(seed, Hkv, G, P, budget, sink, recent):
    rng = np.random.default_rng(seed)
    d = 5
    keys = rng.standard_normal((Hkv, P, d))
    q = rng.standard_normal((Hkv * G, d))
    kept, imp = prefill_keep(keys, q, budget, sink, recent)
    assert kept.tolist() == _brute_prefill_keep(keys.tolist(), q.tolist(), budget, sink, recent)
    np.testing.assert_allclose(imp.sum(axis=1), G, rtol=0, atol=1e-12)  # weights of each head sum to 1


def test_prefill_keep_integer_logits_and_ties():
    # G = 1, small-integer q and k: logits are exact integers, so the kept middle
    # positions are the largest logits, the lower position first on equal ones
    rng = np.random.default_rng(5)
    P, d, budget, sink, recent = 40, 3, 16, 2, 4
    keys = rng.integers(-2, 3, size=(1, P, d)).astype(np.float32)
    q = np.array([[1.0, -1.0, 2.0]], dtype=np.float32)
    kept, _ = prefill_keep(keys, q, budget, sink, recent)
    logit = keys[0] @ q[0]
    middle = sorted(range(sink, P - recent), key=lambda i: (-logit[i], i))[: budget - sink - recent]
    assert kept[0].tolist() == sorted(list(range(sink)) + middle + list(range(P - recent, P)))
    assert len(set(logit[sink:P - recent].tolist())) < P - sink - recent  # ties present and decided by position
