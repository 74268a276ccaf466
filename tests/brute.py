"""Pure-Python brute-force decode step for tiny shapes (no numpy in the arithmetic).

It keeps the cache as a Python list of (position, key, value) tuples per
(sequence, KV head), computes every softmax weight with math.exp, and finds the
victim by scanning all candidates.  It exists to cross-check the numpy oracle on
inputs small enough for loops."""
from __future__ import annotations

import math


class BruteCache:
    def __init__(self, k, v, pos, t, budget, n_q_heads, sink, recent, scale, vl1=False):
        self.B = len(k)
        self.Hkv = len(k[0])
        self.G = n_q_heads // self.Hkv
        self.sink, self.recent, self.scale, self.vl1 = sink, recent, scale, vl1
        self.budget = list(budget)
        self.t = list(t)
        # entries[b][g] = list of [position, key list, value list], index = slot
        self.entries = []
        for b in range(self.B):
            per_g = []
            for g in range(self.Hkv):
                per_g.append([[int(pos[b][i]), [float(x) for x in k[b][g][i]], [float(x) for x in v[b][g][i]]]
                              for i in range(len(pos[b]))])
            self.entries.append(per_g)

    def step(self, q, k_new, v_new):
        """Returns (out[b][h][:], slot[b][g], evicted[b][g] or -1)."""
        outs, slots, evs = [], [], []
        for b in range(self.B):
            t = self.t[b]
            ob, sb, eb = [], [], []
            for g in range(self.Hkv):
                ent = self.entries[b][g]
                keys = [e[1] for e in ent] + [list(map(float, k_new[b][g]))]
                vals = [e[2] for e in ent] + [list(map(float, v_new[b][g]))]
                importance = [0.0] * len(ent)
                for j in range(self.G):
                    qh = list(map(float, q[b][g * self.G + j]))
                    logits = [self.scale * sum(a * c for a, c in zip(qh, kk)) for kk in keys]
                    top = max(logits)
                    w = [math.exp(x - top) for x in logits]
                    z = sum(w)
                    w = [x / z for x in w]
                    o = [sum(w[i] * vals[i][c] for i in range(len(vals))) for c in range(len(qh))]
                    ob.append(o)
                    for i in range(len(ent)):
                        importance[i] += w[i]
                if self.vl1:
                    importance = [importance[i] * sum(abs(x) for x in ent[i][2]) for i in range(len(ent))]
                if len(ent) < self.budget[b]:
                    slot, ev = len(ent), -1
                    ent.append(None)
                else:
                    best, slot = None, None
                    for i in range(len(ent)):
                        p = ent[i][0]
                        if p < self.sink or p >= t - self.recent:
                            continue
                        if best is None or importance[i] < best:
                            best, slot = importance[i], i
                    ev = slot
                ent[slot] = [t, list(map(float, k_new[b][g])), list(map(float, v_new[b][g]))]
                sb.append(slot)
                eb.append(ev)
            outs.append(ob)
            slots.append(sb)
            evs.append(eb)
            self.t[b] = t + 1
        return outs, slots, evs

    def gaps(self, q, k_new, v_new):
        """Per (b, g): second-lowest minus lowest importance over the eligible
        cached entries (inf with fewer than two), found by scanning; no state change."""
        out = []
        for b in range(self.B):
            t = self.t[b]
            row = []
            for g in range(self.Hkv):
                ent = self.entries[b][g]
                keys = [e[1] for e in ent] + [list(map(float, k_new[b][g]))]
                imp = [0.0] * len(ent)
                for j in range(self.G):
                    qh = list(map(float, q[b][g * self.G + j]))
                    logits = [self.scale * sum(a * c for a, c in zip(qh, kk)) for kk in keys]
                    top = max(logits)
                    w = [math.exp(x - top) for x in logits]
                    z = sum(w)
                    for i in range(len(ent)):
                        imp[i] += w[i] / z
                if self.vl1:
                    imp = [imp[i] * sum(abs(x) for x in ent[i][2]) for i in range(len(ent))]
                lowest = second = math.inf
                for i in range(len(ent)):
                    p = ent[i][0]
                    if p < self.sink or p >= t - self.recent:
                        continue
                    if imp[i] < lowest:
                        lowest, second = imp[i], lowest
                    elif imp[i] < second:
                        second = imp[i]
                row.append(second - lowest if second < math.inf else math.inf)
            out.append(row)
        return out

    def positions(self, b, g):
        return [e[0] for e in self.entries[b][g]]
