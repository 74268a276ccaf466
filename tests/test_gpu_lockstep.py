"""Full-length lockstep parity on the four GPU workloads (the oracle follows a
subset of sequences through every decode step of the workload):
  llama8b_b8      sequences 0 and 7, 4096 steps
  throughput_b64  sequences 0 and 63, 16384 steps
  evict_stress    sequences 0-3, 8192 steps (all 16 anchor events)
  ragged_b128     sequence 0 and the sequences of the smallest and the largest
                  budget, 2048 steps
Every step: attention output within tolerance, evicted slot exact or an
accepted tie; every 256 steps the exported importances and log-normalisers;
at the end the recorded sequences' K/V rows bit-for-bit.  Recording runs on
the GPU, the replays in spawned float64 oracle processes (tests/lockstep.py)."""
from __future__ import annotations

import numpy as np
import pytest

from workloads import budgets, get_workload

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

DBG_EVERY = 256


def _plan():
    rag = budgets(get_workload("ragged_b128"))
    lo, hi = int(np.argmin(rag)), int(np.argmax(rag))
    return {
        "llama8b_b8": ([0, 7], 4096),
        "throughput_b64": ([0, 63], 16384),
        "evict_stress": ([0, 1, 2, 3], 8192),
        "ragged_b128": (sorted({0, lo, hi}), 2048),
    }


@pytest.fixture(scope="module")
def lockstep_results(tmp_path_factory, request):
    from lockstep import record, replay_all, set_reporter

    capman = request.config.pluginmanager.getplugin("capturemanager")

    def say(msg):
        with capman.global_and_fixture_disabled():
            print(msg, flush=True)

    set_reporter(say)

    out_dir = str(tmp_path_factory.mktemp("lockstep"))
    jobs = []
    for name, (seqs, steps) in _plan().items():
        assert steps == get_workload(name).decode_steps
        for b, path in zip(seqs, record(name, seqs, steps, DBG_EVERY, out_dir)):
            jobs.append(dict(workload=name, seq=b, steps=steps, dbg_every=DBG_EVERY, path=path,
                             progress=f"{path}.progress"))
    results = replay_all(jobs, workers=16)
    for r in sorted(results, key=lambda r: (r["workload"], r["seq"])):
        say(f"[lockstep] {r['workload']} seq {r['seq']}: {r['steps']} steps, {r['exempt_ties']} accepted ties, "
            f"max out err {r['max_out_err']:.2e}, max score err {r['max_score_err']:.2e}, "
            f"max lse err {r['max_lse_err']:.2e}, {r['dbg_steps']} debug steps, {r['anchor_steps']} anchor events"
            + (f", attention on cached anchors at the events {r['anchor_mass']:.3f}, "
               f"anchors cached at the end {r['anchors_kept']:.1f} of {get_workload(r['workload']).anchors}"
               if r["anchor_mass"] is not None else ""))
    set_reporter(None)
    return {(r["workload"], r["seq"]): r for r in results}


@pytest.mark.parametrize("name", ["llama8b_b8", "throughput_b64", "evict_stress", "ragged_b128"])
def test_full_length_lockstep(lockstep_results, name):
    seqs, steps = _plan()[name]
    for b in seqs:
        r = lockstep_results[(name, b)]
        assert r["error"] is None, f"{name} sequence {b}: {r['error']}"
        assert r["steps"] == steps
        assert r["dbg_steps"] == (steps + DBG_EVERY - 1) // DBG_EVERY
    if name == "evict_stress":
        assert all(lockstep_results[(name, b)]["anchor_steps"] == 16 for b in seqs)
