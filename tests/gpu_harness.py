"""GPU-vs-oracle parity driver shared by the GPU tests.

The HIP library runs the whole batch every step (the launch configuration the
benchmark times); the float64 oracle follows a subset of sequences, which is
exact because sequences are independent.  Each step compares the attention
output element by element and the evicted slot exactly; where the oracle's two
lowest eligible scores are closer than 1e-6 (the agreed exemption) the GPU's
choice is accepted if the oracle rates it eligible and within 1e-6 of its
minimum, and the oracle then takes the GPU's slot (lockstep)."""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np
import torch

from kv_cache_eviction_lf_amd import LongFlowCache
from oracle import SCORE_ATTN, SCORE_NONE, SCORE_VL1, TIE_TOLERANCE, OracleCache
from workloads import Workload, initial_sequence
from workloads.device import device_cache, device_step

TIE_EXEMPTION = TIE_TOLERANCE


def out_tolerance(w: Workload) -> float:
    return 2e-2 if w.dtype == "bf16" else 1e-5


@dataclass
class ParityReport:
    steps: int = 0
    compared_slots: int = 0
    exempt_ties: int = 0
    max_out_err: float = 0.0
    max_score_err: float = 0.0
    max_lse_err: float = 0.0
    diverged_at: int | None = None
    deferred: int = 0  # split chunks that stopped waiting for their pair
    notes: list = field(default_factory=list)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def parity_run(w: Workload, steps: int, check=None, score: str = "attn", chunk_slots: int = 0,
               dbg_every: int = 0, free_running: bool = False, device="cuda:0", max_budget=None,
               compare_cache: bool = True, tag: str = "", split_wait_us=None) -> ParityReport:
    device = torch.device(device)
    check = list(range(w.batch)) if check is None else list(check)
    log(f"[parity{tag}] {w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
        f"{w.dtype} budgets=[{w.budget_lo},{w.budget_hi}] sink={w.sink} recent={w.recent} score={score} "
        f"chunk={chunk_slots} steps={steps} check={check[:8]}{'...' if len(check) > 8 else ''}")
    K, V, seq_len, bud = device_cache(w, device, max_budget=max_budget)
    cache = LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud, score=score,
                          chunk_slots=chunk_slots)
    if split_wait_us is not None:
        cache.set_split_wait(split_wait_us)
    init = [initial_sequence(w, b) for b in check]
    oc = OracleCache([x[0] for x in init], [x[1] for x in init], [x[2] for x in init], [x[3] for x in init],
                     bud[check], w.n_q_heads, w.sink, w.recent,
                     score={"vl1": SCORE_VL1, "none": SCORE_NONE}.get(score, SCORE_ATTN))
    tol = out_tolerance(w)
    rep = ParityReport()
    idx = torch.tensor(check, device=device)
    scores_t = torch.zeros((w.batch, w.n_kv_heads, cache.max_budget), dtype=torch.float32, device=device)
    lse_t = torch.zeros((w.batch, w.n_q_heads), dtype=torch.float32, device=device)
    for s in range(steps):
        (qd, kd, vd), (q, kn, vn) = device_step(w, s, device)
        dbg = dbg_every and s % dbg_every == 0
        if dbg:
            out, ev = cache.step(qd, kd, vd, scores=scores_t, lse=lse_t)
        else:
            out, ev = cache.step(qd, kd, vd)
        out_h = out.index_select(0, idx).float().cpu().numpy().astype(np.float64)
        ev_h = ev.index_select(0, idx).cpu().numpy().astype(np.int64)
        dec = oc.decide(q[check], kn[check], vn[check])
        err = float(np.abs(out_h - dec.out).max())
        rep.max_out_err = max(rep.max_out_err, err)
        assert err <= tol, f"step {s}: attention output differs by {err:.3e} > {tol:.0e}"
        if dbg:
            sc_h = scores_t.index_select(0, idx).cpu().numpy()
            for j, b in enumerate(check):
                n = oc.n[j]
                d_ = np.abs(sc_h[j, :, :n] - dec.scores[j]) / np.maximum(1.0, np.abs(dec.scores[j]))
                rep.max_score_err = max(rep.max_score_err, float(d_.max()) if n else 0.0)
            lse_h = lse_t.index_select(0, idx).cpu().numpy()
            rep.max_lse_err = max(rep.max_lse_err, float(np.abs(lse_h - dec.lse).max()))
            assert rep.max_score_err < 1e-5, f"step {s}: importance differs by {rep.max_score_err:.3e}"
            assert rep.max_lse_err < 1e-4, f"step {s}: lse differs by {rep.max_lse_err:.3e}"
        slots = dec.slot.copy()
        for j in range(len(check)):
            for g in range(w.n_kv_heads):
                ge, oe = int(ev_h[j, g]), int(dec.evict[j, g])
                rep.compared_slots += 1
                if ge == oe:
                    continue
                assert dec.accepts(j, g, ge), (f"step {s} seq {check[j]} kv {g}: GPU evicted {ge}, "
                                               f"oracle {oe} (gap {dec.gap[j, g]:.3e})")
                rep.exempt_ties += 1
                if free_running:
                    rep.diverged_at = s
                slots[j, g] = ge
        if free_running and rep.diverged_at is not None:
            rep.steps = s + 1
            rep.notes.append(f"free-running comparison stopped at exempt tie, step {s}")
            break
        oc.commit(slots, kn[check], vn[check])
        rep.steps = s + 1
    if compare_cache and rep.diverged_at is None:
        Kh = K.index_select(0, idx).float().cpu().numpy()
        Vh = V.index_select(0, idx).float().cpu().numpy()
        for j in range(len(check)):
            nb = oc.budget[j]
            assert np.array_equal(Kh[j, :, :nb], oc.k[j]), f"K cache of sequence {check[j]} differs"
            assert np.array_equal(Vh[j, :, :nb], oc.v[j]), f"V cache of sequence {check[j]} differs"
    st = cache.check_state()  # invariants of the state after the run
    rep.deferred = st.deferred
    cache.close()
    log(f"[parity{tag}] ok: {rep}")
    return rep
