"""Full-length lockstep parity driver (GPU side).

The HIP library runs a workload's whole batch for all of its decode steps, in
the configuration the benchmark times; for a subset of sequences every step's
attention output and evicted slots are recorded on the device (and, every
`dbg_every` steps, the exported importances and log-normalisers), and at the
end their K/V rows.  The other sequences take inputs of the same distribution
from a device pool, which leaves the recorded ones untouched (sequences are
independent); the recorded ones take exactly the seeded step inputs the
oracle uses.  Spawned float64 oracle workers (tests/lockstep_replay.py) then
replay each recorded sequence step by step.  Recording first and replaying
after is the same lockstep: the HIP path never depends on the oracle, and a
replay takes the GPU's slot wherever it accepts a tie."""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

from kv_cache_eviction_lf_amd import LongFlowCache
from workloads import get_workload, step_inputs
from workloads.device import device_cache, device_step_pool, torch_dtype


_reporter = None


def set_reporter(fn) -> None:
    """Where progress lines go (the test passes one that bypasses pytest's
    output capture, so that long runs stay visibly alive)."""
    global _reporter
    _reporter = fn


def note(msg: str) -> None:
    if _reporter is not None:
        _reporter(msg)
    else:
        print(msg, file=sys.stderr, flush=True)


def record(name: str, seqs, steps: int, dbg_every: int, out_dir: str, device="cuda:0", pool_steps: int = 16):
    """Runs `steps` decode steps of workload `name` on the GPU and saves, per
    recorded sequence b, `out_dir/<name>_<b>.npz` with out [steps][Hq][d] (bf16
    bits or fp32), evict [steps][Hkv], scores [n_dbg][Hkv][max_budget], lse
    [n_dbg][Hq] and the final k/v rows [Hkv][max_budget][d].  Returns the paths."""
    dev = torch.device(device)
    w = get_workload(name)
    seqs = [int(b) for b in seqs]
    K, V, seq_len, bud = device_cache(w, dev)
    cache = LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud)
    pool = device_step_pool(w, pool_steps, dev)
    dt = torch_dtype(w)
    idx = torch.tensor(seqs, device=dev)
    ns = len(seqs)
    out_rec = torch.empty((steps, ns, w.n_q_heads, w.head_dim), dtype=dt, device=dev)
    ev_rec = torch.empty((steps, ns, w.n_kv_heads), dtype=torch.int32, device=dev)
    n_dbg = (steps + dbg_every - 1) // dbg_every if dbg_every else 0
    sc_rec = torch.empty((max(n_dbg, 1), ns, w.n_kv_heads, cache.max_budget), dtype=torch.float32, device=dev)
    lse_rec = torch.empty((max(n_dbg, 1), ns, w.n_q_heads), dtype=torch.float32, device=dev)
    scores = torch.zeros((w.batch, w.n_kv_heads, cache.max_budget), dtype=torch.float32, device=dev)
    lse = torch.zeros((w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dt, device=dev)
    ev = torch.empty((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev)
    q = torch.empty_like(out)
    kn = torch.empty((w.batch, w.n_kv_heads, w.head_dim), dtype=dt, device=dev)
    vn = torch.empty_like(kn)
    note(f"[lockstep] {name}: recording sequences {seqs} over {steps} steps")
    t0 = time.time()
    for s in range(steps):
        pq, pk, pv = pool[s % pool_steps]
        q.copy_(pq)
        kn.copy_(pk)
        vn.copy_(pv)
        xq, xk, xv = step_inputs(w, s, seqs)  # the recorded sequences' exact inputs
        q[idx] = torch.from_numpy(xq).to(dt).to(dev)
        kn[idx] = torch.from_numpy(xk).to(dt).to(dev)
        vn[idx] = torch.from_numpy(xv).to(dt).to(dev)
        if dbg_every and s % dbg_every == 0:
            cache.step(q, kn, vn, out=out, evict_idx=ev, scores=scores, lse=lse)
            j = s // dbg_every
            sc_rec[j] = scores.index_select(0, idx)
            lse_rec[j] = lse.index_select(0, idx)
        else:
            cache.step(q, kn, vn, out=out, evict_idx=ev)
        out_rec[s] = out.index_select(0, idx)
        ev_rec[s] = ev.index_select(0, idx)
        if (s + 1) % 2048 == 0:
            torch.cuda.synchronize(dev)
            note(f"[lockstep] {name}: {s + 1}/{steps} steps recorded ({time.time() - t0:.0f} s)")
    torch.cuda.synchronize(dev)
    rep = cache.check_state()
    cache.close()
    bits = (lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)) if dt == torch.bfloat16 else \
        (lambda x: x.cpu().numpy())
    out_h, ev_h = bits(out_rec), ev_rec.cpu().numpy()
    sc_h, lse_h = sc_rec.cpu().numpy(), lse_rec.cpu().numpy()
    k_h, v_h = bits(K.index_select(0, idx)), bits(V.index_select(0, idx))
    paths = []
    for j, b in enumerate(seqs):
        p = os.path.join(out_dir, f"{name}_{b}.npz")
        np.savez(p, out=out_h[:, j], evict=ev_h[:, j], scores=sc_h[:, j], lse=lse_h[:, j], k_final=k_h[j],
                 v_final=v_h[j])
        paths.append(p)
    note(f"[lockstep] {name}: recorded in {time.time() - t0:.0f} s, {rep.deferred} deferred chunks")
    return paths


def replay_all(jobs, workers: int, poll_s: float = 30.0):
    """Runs the replay jobs in spawned oracle processes (no GPU in them), with a
    progress line every `poll_s` seconds from the workers' step counters."""
    from lockstep_replay import replay

    ctx = mp.get_context("spawn")
    env_threads = os.environ.get("OMP_NUM_THREADS")
    os.environ["OMP_NUM_THREADS"] = "1"  # each worker one core; inherited at spawn
    try:
        with ctx.Pool(min(workers, len(jobs))) as pool:
            pending = [(j, pool.apply_async(replay, (j,))) for j in jobs]
            results = []
            t0 = time.time()
            while pending:
                pending[0][1].wait(poll_s)
                still = []
                for j, r in pending:
                    if r.ready():
                        res = r.get()
                        results.append(res)
                        note(f"[lockstep] replayed {res['workload']} seq {res['seq']}: {res['steps']} steps, "
                             f"{res['exempt_ties']} ties, {res['seconds']:.0f} s, "
                             f"{'ok' if res['error'] is None else res['error']}")
                    else:
                        still.append((j, r))
                pending = still
                if pending:
                    prog = []
                    for j, _ in pending:
                        try:
                            prog.append(f"{j['workload']}:{j['seq']}@{open(j['progress']).read().split()[0]}")
                        except (OSError, IndexError):
                            prog.append(f"{j['workload']}:{j['seq']}@0")
                    note(f"[lockstep] {time.time() - t0:.0f} s, replaying " + " ".join(prog))
            return results
    finally:
        if env_threads is None:
            os.environ.pop("OMP_NUM_THREADS", None)
        else:
            os.environ["OMP_NUM_THREADS"] = env_threads
