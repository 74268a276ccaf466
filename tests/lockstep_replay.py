"""Replay of one recorded sequence through the float64 oracle (worker side of
tests/lockstep.py).  Imports numpy, the oracle and the input recipes only: it
runs in a spawned process that never touches the GPU.

For every step the oracle decides from the same seeded inputs the HIP path
received, and the recorded GPU result must match: the attention output within
the dtype's tolerance, the evicted slot exactly or, where the oracle's two
lowest eligible importances are closer than the tie tolerance, a slot the
oracle accepts (the oracle then takes the GPU's slot, so both caches stay
identical).  On recorded debug steps the exported importances and
log-normalisers are compared too, and at the end the sequence's K/V rows
bit-for-bit."""
from __future__ import annotations

import os
import time

import numpy as np


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def replay(job: dict) -> dict:
    from threadpoolctl import threadpool_limits

    from oracle import OracleCache, TIE_TOLERANCE
    from workloads import anchor_event, anchor_positions, budgets, get_workload, initial_sequence, step_inputs

    w = get_workload(job["workload"])
    b, steps, dbg_every = job["seq"], job["steps"], job["dbg_every"]
    rec = np.load(job["path"])
    bf16 = w.dtype == "bf16"
    tol = 2e-2 if bf16 else 1e-5
    out = rec["out"]
    ev = rec["evict"]
    k, v, pos, t = initial_sequence(w, b)
    bud = int(budgets(w)[b])
    res = dict(workload=w.name, seq=b, steps=0, exempt_ties=0, max_out_err=0.0, max_score_err=0.0,
               max_lse_err=0.0, dbg_steps=0, anchor_steps=0, anchor_mass=None, anchors_kept=None, error=None)
    progress = job.get("progress")
    # Diagnostics of the anchor workload (the caches are the GPU's: the replay
    # follows its evictions): the share of the group's attention that lands on
    # cached anchor tokens at the anchor events, and how many anchors are still
    # cached at the end.
    anchor_pos = anchor_positions(w, bud) if w.anchors else None
    mass = []
    t0 = time.time()
    with threadpool_limits(1):
        oc = OracleCache([k], [v], [pos], [t], bud, w.n_q_heads, w.sink, w.recent)
        for s in range(steps):
            q, kn, vn = step_inputs(w, s, [b])
            dec = oc.decide(q, kn, vn)
            got = _bf16_to_f32(out[s]) if bf16 else out[s]
            err = float(np.abs(got.astype(np.float64) - dec.out[0]).max())
            res["max_out_err"] = max(res["max_out_err"], err)
            if err > tol:
                res["error"] = f"step {s}: attention output differs by {err:.3e} > {tol:.0e}"
                break
            if dbg_every and s % dbg_every == 0:
                j = s // dbg_every
                n = oc.n[0]
                sc = rec["scores"][j][:, :n].astype(np.float64)
                d_ = np.abs(sc - dec.scores[0]) / np.maximum(1.0, np.abs(dec.scores[0]))
                res["max_score_err"] = max(res["max_score_err"], float(d_.max()) if n else 0.0)
                res["max_lse_err"] = max(res["max_lse_err"], float(np.abs(rec["lse"][j] - dec.lse[0]).max()))
                res["dbg_steps"] += 1
                if res["max_score_err"] >= 1e-5 or res["max_lse_err"] >= 1e-4:
                    res["error"] = (f"step {s}: importance differs by {res['max_score_err']:.3e}, "
                                    f"lse by {res['max_lse_err']:.3e}")
                    break
            slots = dec.slot.copy()
            bad = None
            for g in range(w.n_kv_heads):
                ge, oe = int(ev[s, g]), int(dec.evict[0, g])
                if ge == oe:
                    continue
                if not dec.accepts(0, g, ge, TIE_TOLERANCE):
                    bad = f"step {s} kv {g}: GPU evicted {ge}, oracle {oe} (gap {dec.gap[0, g]:.3e})"
                    break
                res["exempt_ties"] += 1
                slots[0, g] = ge
            if bad:
                res["error"] = bad
                break
            if anchor_pos is not None and anchor_event(w, s) is not None:
                n = oc.n[0]
                on = np.isin(oc.pos[0][:, :n], anchor_pos)
                mass.append(float((dec.scores[0] * on).sum() / (w.group * w.n_kv_heads)))
            oc.commit(slots, kn, vn)
            res["steps"] = s + 1
            res["anchor_steps"] += anchor_event(w, s) is not None
            if progress and (s + 1) % 512 == 0:
                with open(progress, "w") as f:
                    f.write(f"{s + 1} {time.time() - t0:.1f}\n")
    if anchor_pos is not None:
        res["anchor_mass"] = float(np.mean(mass)) if mass else None
        res["anchors_kept"] = float(np.isin(oc.pos[0][:, :oc.n[0]], anchor_pos).sum() / w.n_kv_heads)
    if res["error"] is None:
        kf, vf = rec["k_final"], rec["v_final"]
        if bf16:
            kf, vf = _bf16_to_f32(kf), _bf16_to_f32(vf)
        if not (np.array_equal(kf[:, :bud].astype(np.float64), oc.k[0]) and
                np.array_equal(vf[:, :bud].astype(np.float64), oc.v[0])):
            res["error"] = "final K/V rows differ from the oracle's cache"
    if progress:
        with open(progress, "w") as f:
            f.write(f"{res['steps']} {time.time() - t0:.1f} done\n")
    res["seconds"] = time.time() - t0
    return res
