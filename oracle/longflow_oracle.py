"""Float64 CPU oracle of one LongFlow decode step.

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU-baseline
leg may import this module; the HIP library never does, and this module uses
nothing from it.

What one step computes, for every sequence b and KV head g of a static,
fixed-budget cache (the LongFlow summary, gist.science, section 2.C: a
statically pre-allocated KV cache and one fused operator doing attention,
importance estimation and eviction; the LongFlow blog post, denisavetisyan.com,
figure caption on the dataflow: attention output O and score I are produced
from the intermediates S and P while KV blocks and a mask stream in):

1. Decode attention of each query head h of the group over the cached tokens
   plus the incoming token: alpha = softmax(scale * K q_h), o_h = alpha V
   (standard scaled-dot-product attention, scale = 1/sqrt(d) unless given).
2. Importance of every cached slot, from the current query only (zero-history
   estimation, summary section 2.A) and from the weights attention has just
   produced (zero-cost estimation, summary section 2.A):
     SCORE_ATTN: I_i = sum over the group's query heads of alpha_{h,i}
     SCORE_VL1 : I_i = (sum_h alpha_{h,i}) * sum_l |v_i[l]|, the L1 norm of the
                 contribution vector alpha_i v_i of the LongFlowScore equation
                 (summary section 2.B), summed over the group's heads.
   alpha keeps the denominator of this step; nothing is renormalised after the
   eviction (summary section 2.B, denominator approximation).
3. Slots holding the first ``sink`` positions and the ``recent`` newest cached
   positions are not candidates; the incoming token is never a candidate.
4. The candidate with the smallest importance is evicted (summary section 2.B:
   remove the token whose removal perturbs attention least); on equal scores
   the lowest slot index wins.
5. The incoming token's K/V overwrite that slot (blog figure caption: one token
   evicted after each attention computation).  While the cache is not yet full
   the token is appended to the next free slot instead and nothing is evicted.

Readings where the pages are silent (also listed in the design notes): query
head h belongs to KV head h // G (contiguous groups); eviction is per
(sequence, KV head); the score sums the G query heads of the group.

Representation: unlike the HIP path (which keeps a ring of recent slots), the
oracle stores the absolute position held by every slot and derives the
protected set from positions.  K/V are held in float64 (exact for the fp32 and
bf16 inputs it receives).

Pins (tests/test_oracle_pins.py, tests/golden/): torch's float64
scaled_dot_product_attention with GQA on caches that never evict; a hand-worked
two-head example with rational weights (tests/golden/hand_worked_step.json);
uniform keys (closed-form weights 1/(n+1) and first-slot tie-break); weights of
each head summing to 1; G=1 integer logits where the argmin is the argmin of
the logit; the StreamingLLM-like closed form of the kept set when logits rise
with position; VL1 equal to the L1 norm of the output change when one token's
contribution is removed; brute-force pure-Python steps on tiny shapes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SCORE_ATTN = 0
SCORE_VL1 = 1
# Full-cache comparator (the uncompressed cache the LongFlow summary, section
# 3, compares against): attention only, no importance and no eviction.  The
# incoming token is appended while there is room; once the cache is full it is
# attended but not stored (a reading: the pages' full cache never fills).
SCORE_NONE = 2
# Importances closer than this are a tie: either slot is a correct eviction.
TIE_TOLERANCE = 1e-6


def attention_step(keys: np.ndarray, values: np.ndarray, q_heads: np.ndarray, scale: float):
    """Softmax attention of every row of ``q_heads`` over ``keys``/``values``.

    keys, values: float64 [n][d]; q_heads: float64 [G][d].
    Returns (alpha [G][n], out [G][d], lse [G]) with lse the natural-log
    normaliser log(sum_i exp(scale q.k_i))."""
    s = scale * (q_heads @ keys.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    alpha = e / z
    return alpha, alpha @ values, m[:, 0] + np.log(z[:, 0])


@dataclass
class StepDecision:
    out: np.ndarray  # float64 [B][Hq][d]
    slot: np.ndarray  # int64 [B][Hkv]: slot receiving the incoming token
    evict: np.ndarray  # int64 [B][Hkv]: evicted slot, -1 when appended
    scores: list  # per sequence: float64 [Hkv][n_b], importance of every cached slot
    eligible: list  # per sequence: bool [Hkv][n_b], slot may be evicted
    gap: np.ndarray  # float64 [B][Hkv]: 2nd lowest - lowest eligible score (inf if < 2)
    alpha_new: np.ndarray  # float64 [B][Hq]: weight of the incoming token
    lse: np.ndarray  # float64 [B][Hq]

    def accepts(self, b: int, g: int, slot: int, tol: float = TIE_TOLERANCE) -> bool:
        """Whether ``slot`` is a correct choice for (sequence b, KV head g).

        The oracle's own slot always is.  Where several slots are correct
        answers, namely when the two lowest eligible importances are closer
        than ``tol``, another slot is also accepted if it is eligible and its
        importance is within ``tol`` of the lowest one.  Anything else (an
        appended token in the wrong place, a protected slot, a clearly larger
        importance) is rejected."""
        want = int(self.evict[b, g])
        slot = int(slot)
        if slot == want:
            return True
        if want < 0 or slot < 0 or not self.gap[b, g] < tol:
            return False
        el, sc = self.eligible[b][g], self.scores[b][g]
        return slot < el.shape[0] and bool(el[slot]) and sc[slot] - sc[want] < tol


class OracleCache:
    """One layer's static cache for a batch of sequences, as the oracle tracks it.

    k, v: per sequence float arrays [Hkv][n_b][d] holding the n_b cached tokens
    in slots 0..n_b-1; pos: per sequence int arrays [n_b] (or [Hkv][n_b]) with
    the absolute position of each of them; t: per sequence, position of the
    next incoming token; budget: per sequence slot budget (n_b <= budget_b)."""

    def __init__(self, k, v, pos, t, budget, n_q_heads, sink, recent, scale=None, score=SCORE_ATTN):
        nb = len(k)
        self.B = nb
        self.Hkv, _, self.d = np.asarray(k[0]).shape
        self.Hq = int(n_q_heads)
        if self.Hq % self.Hkv:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        self.G = self.Hq // self.Hkv
        self.sink = int(sink)
        self.recent = int(recent)
        self.scale = float(1.0 / np.sqrt(self.d) if scale is None else scale)
        self.score = int(score)
        self.budget = [int(x) for x in np.broadcast_to(np.asarray(budget), (nb,))]
        self.k, self.v, self.pos, self.n = [], [], [], []
        for b in range(nb):
            kb = np.asarray(k[b], dtype=np.float64)
            vb = np.asarray(v[b], dtype=np.float64)
            n = kb.shape[1]
            if n > self.budget[b]:
                raise ValueError("more cached tokens than the budget")
            if self.budget[b] <= self.sink + self.recent:
                raise ValueError("budget must exceed sink + recent")
            K = np.zeros((self.Hkv, self.budget[b], self.d))
            V = np.zeros_like(K)
            K[:, :n] = kb
            V[:, :n] = vb
            P = np.full((self.Hkv, self.budget[b]), -1, dtype=np.int64)
            P[:, :n] = np.broadcast_to(np.asarray(pos[b], dtype=np.int64), (self.Hkv, n))
            self.k.append(K)
            self.v.append(V)
            self.pos.append(P)
            self.n.append(n)
        self.t = [int(x) for x in np.asarray(t).reshape(-1)]

    def decide(self, q, k_new, v_new) -> StepDecision:
        """Attention, importance and the slot choice for one step (no state change)."""
        q = np.asarray(q, dtype=np.float64)
        k_new = np.asarray(k_new, dtype=np.float64)
        v_new = np.asarray(v_new, dtype=np.float64)
        B, Hkv, G, d = self.B, self.Hkv, self.G, self.d
        out = np.zeros((B, self.Hq, d))
        slot = np.zeros((B, Hkv), dtype=np.int64)
        evict = np.zeros((B, Hkv), dtype=np.int64)
        gap = np.full((B, Hkv), np.inf)
        alpha_new = np.zeros((B, self.Hq))
        lse = np.zeros((B, self.Hq))
        scores, eligible = [], []
        for b in range(B):
            n, t = self.n[b], self.t[b]
            sc = np.zeros((Hkv, n))
            el = np.zeros((Hkv, n), dtype=bool)
            for g in range(Hkv):
                keys = np.concatenate([self.k[b][g, :n], k_new[b, g][None]])
                vals = np.concatenate([self.v[b][g, :n], v_new[b, g][None]])
                heads = slice(g * G, (g + 1) * G)
                alpha, o, l = attention_step(keys, vals, q[b, heads], self.scale)
                out[b, heads] = o
                lse[b, heads] = l
                alpha_new[b, heads] = alpha[:, n]
                if self.score == SCORE_NONE:
                    if n < self.budget[b]:
                        slot[b, g], evict[b, g] = n, -1
                    else:
                        slot[b, g], evict[b, g] = -1, -2  # attended, not stored
                    continue
                imp = alpha[:, :n].sum(axis=0)
                if self.score == SCORE_VL1:
                    imp = imp * np.abs(vals[:n]).sum(axis=1)
                p = self.pos[b][g, :n]
                ok = (p >= self.sink) & (p < t - self.recent)
                sc[g], el[g] = imp, ok
                cand = np.flatnonzero(ok)
                if cand.size >= 2:
                    two = np.sort(imp[cand])[:2]
                    gap[b, g] = two[1] - two[0]
                if n < self.budget[b]:
                    slot[b, g], evict[b, g] = n, -1
                else:
                    if cand.size == 0:
                        raise RuntimeError("full cache with no evictable slot")
                    e = int(cand[np.argmin(imp[cand])])  # argmin returns the first minimum
                    slot[b, g], evict[b, g] = e, e
            scores.append(sc)
            eligible.append(el)
        return StepDecision(out, slot, evict, scores, eligible, gap, alpha_new, lse)

    def commit(self, slot, k_new, v_new):
        """Write the incoming tokens into ``slot`` [B][Hkv] and advance the positions."""
        slot = np.asarray(slot, dtype=np.int64)
        k_new = np.asarray(k_new, dtype=np.float64)
        v_new = np.asarray(v_new, dtype=np.float64)
        for b in range(self.B):
            n, t = self.n[b], self.t[b]
            for g in range(self.Hkv):
                s = int(slot[b, g])
                if s == -1 and self.score == SCORE_NONE and n >= self.budget[b]:
                    continue  # full comparator cache: the token is not stored
                if n < self.budget[b]:
                    if s != n:
                        raise ValueError("a cache that is not full appends at its next free slot")
                else:
                    p = self.pos[b][g, s]
                    if not (0 <= s < self.budget[b]) or p < self.sink or p >= t - self.recent:
                        raise ValueError(f"slot {s} of ({b},{g}) is protected")
                self.k[b][g, s] = k_new[b, g]
                self.v[b][g, s] = v_new[b, g]
                self.pos[b][g, s] = t
            self.t[b] = t + 1
            self.n[b] = min(n + 1, self.budget[b])

    def step(self, q, k_new, v_new) -> StepDecision:
        dec = self.decide(q, k_new, v_new)
        self.commit(dec.slot, k_new, v_new)
        return dec


def prefill_keep(keys, q_last, budget: int, sink: int, recent: int, scale=None):
    """One-shot, history-free compression of a prefill longer than the budget.

    The same importance as the decode step (LongFlow summary, section 2.A: from
    the current query only, a by-product of its attention; the summary's
    section 5 leaves long prefill to other methods, so this is a reading): the
    last prefill query attends over all P prefill tokens, and a token's
    importance is the softmax weight it gets, summed over the query heads of its
    KV group.  Kept per KV head: positions [0, sink), the `recent` last
    positions [P - recent, P), and the budget - sink - recent middle positions
    of largest importance (equal importance: the lower position first).

    keys: float [Hkv][P][d]; q_last: float [Hq][d] (query heads grouped
    contiguously).  Returns (kept int64 [Hkv][min(P, budget)] in increasing
    position order, importance float64 [Hkv][P])."""
    keys = np.asarray(keys, dtype=np.float64)
    q_last = np.asarray(q_last, dtype=np.float64)
    Hkv, P, d = keys.shape
    G = q_last.shape[0] // Hkv
    scale = float(1.0 / np.sqrt(d) if scale is None else scale)
    if budget <= sink + recent:
        raise ValueError("budget must exceed sink + recent")
    imp = np.zeros((Hkv, P))
    kept = []
    for g in range(Hkv):
        alpha, _, _ = attention_step(keys[g], keys[g], q_last[g * G:(g + 1) * G], scale)
        imp[g] = alpha.sum(axis=0)
        if P <= budget:
            kept.append(np.arange(P))
            continue
        middle = list(range(sink, P - recent))
        ranked = sorted(middle, key=lambda i: (-imp[g, i], i))[: budget - sink - recent]
        kept.append(np.array(sorted(list(range(sink)) + ranked + list(range(P - recent, P)))))
    return np.stack(kept).astype(np.int64), imp
