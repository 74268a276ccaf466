"""Benchmark of the fused LongFlow decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b_b8]

A step is one lf_decode_step over the whole batch of one layer cache:
attention + importance + argmin + in-place overwrite for every (sequence, KV
head).  Layer caches rotate (L of them, each a separate static cache) so that
the K/V bytes of consecutive steps do not fit in the 256 MB Infinity Cache and
every step streams from HBM.  Steps are captured in HIP graphs and replayed;
the timed region is bracketed by device synchronisation and HIP events on the
launch stream.  Inputs are seeded synthetic data already resident in HBM.

Prints one JSON line (rank 0, N = 1): decode steps/s, the roofline of the
decode kernel (algorithmic bytes per launch / average launch time vs 8 TB/s)
and the float64 CPU oracle timed on a bounded sample of the same workload."""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama8b_b8")
    ap.add_argument("--layers", type=int, default=0, help="rotating layer caches (0 = enough to exceed 2x MALL)")
    ap.add_argument("--score", default="attn", choices=["attn", "vl1", "none"],
                    help="none: the full-cache comparator (attention only, the cache is full and keeps its tokens)")
    ap.add_argument("--compress", action="store_true",
                    help="time the one-shot prefill compression (lf_prefill_compress) of the workload's shape "
                         "instead of decode steps (prefill lengths: the ragged draw, else twice the budget)")
    ap.add_argument("--budget", type=int, default=0,
                    help="override the workload's budget (equal for every sequence, prefill filling it)")
    ap.add_argument("--chunk", type=int, default=0, help="split-KV chunk slots (0 = library default)")
    ap.add_argument("--eager", action="store_true", help="launch step by step instead of replaying HIP graphs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read/copy probes and the launch floor")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the short runs of the other GPU workloads reported under 'workloads'")
    ap.add_argument("--other-steps", type=int, default=1000, help="timed steps of each other workload")
    return ap.parse_args()


OTHER_WORKLOADS = ("llama8b_b8", "throughput_b64", "evict_stress", "ragged_b128")


def fast_caches(w, bud, L, dev, torch):
    """L layer caches of workload w for timing only: K/V drawn N(0,1) on the
    device (the key outlier channels scaled), filled to each sequence's
    prefill length or budget, instead of the seeded host recipe (whose values
    only parity runs need); prefills longer than the budgets (the ragged
    batch) are drawn at full length and compressed to the budgets."""
    from workloads import prefill_lengths
    from workloads.generate import outlier_channels

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
    ch = torch.as_tensor(outlier_channels(w), device=dev)
    S = int(bud.max())
    seq_len = prefill_lengths(w)
    out = []
    if w.prefill == "ragged":
        # Prefills longer than the budgets, compressed down to them at start by
        # the method's own one-shot compression (lf_prefill_compress): the
        # caches hold the kept tokens of N(0,1) prefills in position order.
        from kv_cache_eviction_lf_amd import compress_prefill

        P = int(seq_len.max())
        for _ in range(L):
            q = torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=gen, device=dev).to(dt)
            k_pre = torch.randn((w.batch, w.n_kv_heads, P, w.head_dim), generator=gen, device=dev).to(dt)
            v_pre = torch.randn((w.batch, w.n_kv_heads, P, w.head_dim), generator=gen, device=dev).to(dt)
            K, V, _, _ = compress_prefill(q, k_pre, v_pre, [int(x) for x in seq_len], S, w.sink, w.recent,
                                          budgets=[int(x) for x in bud])
            del k_pre, v_pre
            out.append((K, V, seq_len))
        torch.cuda.synchronize()
        return out
    for _ in range(L):
        K = torch.randn((w.batch, w.n_kv_heads, S, w.head_dim), generator=gen, device=dev)
        if ch.numel():
            K[..., ch] *= w.outlier_scale
        V = torch.randn((w.batch, w.n_kv_heads, S, w.head_dim), generator=gen, device=dev)
        out.append((K.to(dt), V.to(dt), seq_len))
    return out


def algorithmic_bytes(w, bud, stored: bool = True) -> int:
    """Bytes one step must move: every cached K and V row read, k_new/v_new read
    and (unless a full comparator cache keeps its tokens) written into the victim
    slot, q read and the output written."""
    s = 2 if w.dtype == "bf16" else 4
    kv = int(np.sum(bud)) * w.n_kv_heads * w.head_dim * 2 * s
    new = (2 if stored else 1) * w.batch * w.n_kv_heads * w.head_dim * 2 * s
    qo = 2 * w.batch * w.n_q_heads * w.head_dim * s
    return kv + new + qo


def code_sha256(text: str) -> str:
    """sha256 of C++/HIP source with its comments, trailing blanks and empty
    lines removed: it changes with the code and not with its comments (the
    kernel sources hold no string literal that contains a comment marker)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()


def profiled_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this workload, if it was taken on the current kernel code."""
    path = os.path.join(ROOT, "profiles", f"lf_step_kernel_{workload}_traffic.json")
    src = os.path.join(ROOT, "kv_cache_eviction_lf_amd", "csrc", "lf_kernel.hip")
    try:
        rec = json.load(open(path))
        sha = code_sha256(open(src).read())
    except (OSError, ValueError):
        return None
    return rec.get("traffic_bytes_per_launch") if rec.get("kernel_code_sha256") == sha else None


def host_cores() -> int:
    """CPU cores this process may run on (the box's share, not the machine's)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w, seconds: float, score: str = "attn", threads: int = 0) -> dict:
    """Time the float64 oracle as it stands on the same workload (full batch of
    the first layer) for about `seconds`, with BLAS allowed `threads` threads
    (0 = every host core of this process)."""
    from threadpoolctl import threadpool_limits

    from oracle import SCORE_ATTN, SCORE_NONE, SCORE_VL1, OracleCache
    from workloads import budgets, initial_cache, step_inputs

    threads = threads or host_cores()
    with threadpool_limits(threads):
        ks, vs, ps, ts = initial_cache(w)
        oc = OracleCache(ks, vs, ps, ts, budgets(w), w.n_q_heads, w.sink, w.recent,
                         score={"vl1": SCORE_VL1, "none": SCORE_NONE}.get(score, SCORE_ATTN))
        inputs = [step_inputs(w, s) for s in range(4)]
        oc.step(*inputs[0])  # warm-up
        n, t0 = 0, time.perf_counter()
        while True:
            oc.step(*inputs[(n + 1) % 4])
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds and n >= 2:
                break
    return {"value": n / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name} full batch ({w.batch} sequences), {n} float64 oracle steps after 1 warm-up, "
                      f"{el:.1f} s, numpy with BLAS allowed {threads} thread{'s' if threads > 1 else ''} "
                      f"of the {host_cores()} host cores"}


def bench_compress(args, w, torch, dev):
    """Time lf_prefill_compress over the workload's batch: every sequence's
    prefill (longer than its budget) reduced to its budget."""
    from kv_cache_eviction_lf_amd import _lib
    from workloads import budgets, prefill_lengths

    bud = budgets(w)
    pre = prefill_lengths(w) if w.prefill == "ragged" else 2 * bud.astype(np.int64)
    max_prefill, max_budget = int(pre.max()), int(bud.max())
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    q = torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=gen, device=dev).to(tdt)
    k_pre = torch.randn((w.batch, w.n_kv_heads, max_prefill, w.head_dim), generator=gen, device=dev).to(tdt)
    v_pre = torch.randn_like(k_pre, dtype=torch.float32).to(tdt)
    k_cache = torch.empty((w.batch, w.n_kv_heads, max_budget, w.head_dim), dtype=tdt, device=dev)
    v_cache = torch.empty_like(k_cache)
    kept = torch.empty((w.batch, w.n_kv_heads, max_budget), dtype=torch.int32, device=dev)
    cfg = _lib.make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, max_budget, w.sink, w.recent,
                           _lib.LF_BF16 if w.dtype == "bf16" else _lib.LF_F32)
    wb = _lib.lf_prefill_work_bytes(cfg, max_prefill)
    work = torch.empty(wb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    prel, budl = [int(x) for x in pre], [int(x) for x in bud]

    def once():
        _lib.lf_prefill_compress(cfg, budl, prel, max_prefill, q.data_ptr(), k_pre.data_ptr(), v_pre.data_ptr(),
                                 k_cache.data_ptr(), v_cache.data_ptr(), kept.data_ptr(), work.data_ptr(), wb, stream)

    n = max(3, min(args.steps, 50))
    for _ in range(2):
        once()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        once()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    s = 2 if w.dtype == "bf16" else 4
    nkeep = np.minimum(pre, bud).astype(np.int64)
    # every prefill K row read, the kept K and V rows read and written
    nbytes = int((pre.sum() + 4 * nkeep.sum()) * w.n_kv_heads * w.head_dim * s)
    gbps = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "prefill compressions/s (one-shot, the whole batch to its budgets)",
        "value": round(1e3 / ms, 2), "unit": "compressions/s", "n_gpus": 1, "steps": n, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded torch normal on the device)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "prefill": [int(pre.min()), int(pre.max())],
                   "budget": [int(bud.min()), int(bud.max())], "sink": w.sink, "recent": w.recent},
        "kv_GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_call": nbytes,
        "note": "bytes: every prefill K row read once (the statistics pass stores the logits the selection "
                "pass reads) plus the kept K and V rows read and written",
    }), flush=True)


def time_steps(args, w, bud, steps, warmup, torch, dev, lib, fast=False):
    """Times `steps` decode steps of workload w (after `warmup`) over L rotating
    layer caches; returns (ms per step, wall seconds of the timed region, L,
    chunk slots)."""
    from kv_cache_eviction_lf_amd import LongFlowCache, _lib
    from workloads.device import device_cache, device_step_pool

    layer_kv = int(np.sum(bud)) * w.n_kv_heads * w.head_dim * 2 * (2 if w.dtype == "bf16" else 4)
    L = (args.layers if not fast else 0) or max(1, math.ceil(2 * MALL_BYTES / layer_kv))
    # L independent layer caches (distinct seeds) and fresh inputs for every
    # step (a repeated input would fill the caches with copies of its tokens).
    caches = []
    if fast or w.prefill == "ragged":
        for K, V, seq_len in fast_caches(w, bud, L, dev, torch):
            caches.append(LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud,
                                        score=args.score, chunk_slots=args.chunk))
    else:
        for layer in range(L):
            wl = w.with_(seed=w.seed + 7919 * layer)
            K, V, seq_len, _ = device_cache(wl, dev)
            caches.append(LongFlowCache(K, V, w.n_q_heads, w.sink, w.recent, seq_len, budgets=bud,
                                        score=args.score, chunk_slots=args.chunk))
    step_in = 2 * (w.batch * w.n_q_heads + 2 * w.batch * w.n_kv_heads) * w.head_dim * (2 if w.dtype == "bf16" else 4)
    P = max(1, min(warmup + steps, (16 << 30) // step_in))
    pool = device_step_pool(w, P, dev)
    outs = [torch.empty_like(pool[0][0]) for _ in range(L)]
    evs = [torch.empty((w.batch, w.n_kv_heads), dtype=torch.int32, device=dev) for _ in range(L)]
    ptrs = [(caches[i].handle, outs[i].data_ptr(), evs[i].data_ptr()) for i in range(L)]
    qptrs = [tuple(t.data_ptr() for t in x) for x in pool]
    step_fn = lib.lf_decode_step

    def launch(k, stream):
        h, o, e = ptrs[k % L]
        q, kn, vn = qptrs[k % P]
        st = step_fn(q, kn, vn, h, o, e, stream)
        if st:
            raise RuntimeError(f"lf_decode_step failed: {_lib.lf_last_error()}")

    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()

    def run_eager(n, base):
        sh = cur.cuda_stream
        for k in range(n):
            launch(base + k, sh)

    graphs = {}

    def graph_for(n, base):
        key = (n, base)
        if key not in graphs:
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            with torch.cuda.graph(g, stream=cs):
                sh = torch.cuda.current_stream().cuda_stream
                for k in range(n):
                    launch(base + k, sh)
            graphs[key] = g
        return graphs[key]

    chunk = 512 if not args.eager else 0

    def pieces(n, base):  # graphs of up to `chunk` consecutive steps
        return [(min(chunk, n - i), base + i) for i in range(0, n, chunk)]

    # pre-capture what warm-up and the timed region replay (capture launches nothing)
    if not args.eager:
        for n, b in pieces(warmup, 0) + pieces(steps, warmup):
            graph_for(n, b)

    def run(n, base):
        if args.eager:
            run_eager(n, base)
            return
        for m, b in pieces(n, base):
            graph_for(m, b).replay()

    run(warmup, 0)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(cur)
    run(steps, warmup)
    ev1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / steps
    chunk_slots = caches[0].cfg.chunk_slots or "auto"
    for c in caches:
        c.close()
    return ms_per_step, wall, L, chunk_slots


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode step has no cross-GPU exchange, and this build "
              "runs on a single MI355X; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_eviction_lf_amd import _lib
    from workloads import budgets, get_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = _lib.load_library()
    dev = torch.device("cuda:0")
    w = get_workload(args.workload)
    if args.budget:
        w = w.with_(budget_lo=args.budget, budget_hi=args.budget, prefill="full")
    if args.compress:
        bench_compress(args, w, torch, dev)
        return
    bud = budgets(w)
    step_bytes = algorithmic_bytes(w, bud, stored=args.score != "none")
    ms_per_step, wall, L, chunk_slots = time_steps(args, w, bud, args.steps, args.warmup, torch, dev, lib)
    steps_per_s = 1e3 / ms_per_step
    achieved = step_bytes / (ms_per_step * 1e-3) / 1e9  # GB/s
    others = None
    if not args.no_others and args.score == "attn" and not args.budget and not args.chunk and not args.layers:
        others = {}
        for name in OTHER_WORKLOADS:
            if name == w.name:
                continue
            wo = get_workload(name)
            bo = budgets(wo)
            mo, _, Lo, _ = time_steps(args, wo, bo, args.other_steps, min(args.warmup, 200), torch, dev, lib,
                                      fast=True)
            bo_bytes = algorithmic_bytes(wo, bo)
            gb = bo_bytes / (mo * 1e-3) / 1e9
            others[name] = {"ms_per_step": round(mo, 6), "steps_per_s": round(1e3 / mo, 1), "kv_GBps": round(gb, 1),
                            "frac": round(gb / HBM_PEAK_GBPS, 4), "steps": args.other_steps, "layer_caches": Lo,
                            "bytes_per_launch": bo_bytes}
            if wo.prefill == "ragged":
                others[name]["initial_cache"] = "full-length prefills compressed to the budgets by lf_prefill_compress"

    cur = torch.cuda.current_stream()
    probe = None
    if not args.no_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        sink = torch.empty(_lib.lf_probe_read_sink_words(), dtype=torch.int32, device=dev)
        res = {}
        for name in ("read", "copy"):
            for _ in range(3):
                if name == "read":
                    _lib.lf_probe_read(src.data_ptr(), n, sink.data_ptr(), cur.cuda_stream)
                else:
                    _lib.lf_probe_copy(src.data_ptr(), dst.data_ptr(), n, cur.cuda_stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            for _ in range(10):
                if name == "read":
                    _lib.lf_probe_read(src.data_ptr(), n, sink.data_ptr(), cur.cuda_stream)
                else:
                    _lib.lf_probe_copy(src.data_ptr(), dst.data_ptr(), n, cur.cuda_stream)
            b.record(cur)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 10 * 1e-3
            res[name + "_GBps"] = round((n if name == "read" else 2 * n) / t / 1e9, 1)
        # Launch floor: a graph of empty 256-workgroup launches, replayed the
        # way the steps are (per-node cost before any byte moves).
        nodes = 512
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cs):
            sh = torch.cuda.current_stream().cuda_stream
            for _ in range(nodes):
                _lib.lf_probe_empty(256, sh)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        for _ in range(4):
            g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        res["launch_floor_us"] = round(a.elapsed_time(b) * 1e3 / (4 * nodes), 2)
        # The same read probe over the step's own byte count, one launch per
        # graph node and rotating buffers past the Infinity Cache like the
        # layer caches: what a kernel that only streams the step's bytes takes
        # per launch at this size (ramp and launch included).  Below a few
        # hundred MB the fastest grid depends on the size, so several grids
        # are timed and the fastest is the ceiling.
        del src, dst
        ns = (step_bytes + 15) // 16 * 16
        Lp = max(2, -(-(512 << 20) // ns))
        bufs = [torch.empty(ns, dtype=torch.uint8, device=dev) for _ in range(Lp)]
        nodes = max(8, min(512, (64 << 30) // (ns * 8)))
        per_grid = {}
        for grid in (256, 512, 1024, 2048):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                sh = torch.cuda.current_stream().cuda_stream
                for k in range(nodes):
                    _lib.lf_probe_read_grid(bufs[k % Lp].data_ptr(), ns, grid, sink.data_ptr(), sh)
            g.replay()
            torch.cuda.synchronize()
            a.record(cur)
            for _ in range(3):
                g.replay()
            b.record(cur)
            torch.cuda.synchronize()
            per_grid[grid] = a.elapsed_time(b) * 1e3 / (3 * nodes)
            del g
        best = min(per_grid, key=per_grid.get)
        us = per_grid[best]
        res["read_step_bytes_us"] = round(us, 2)
        res["read_step_bytes_GBps"] = round(ns / us / 1e3, 1)
        res["read_step_bytes_grid"] = best
        res["read_step_bytes_us_by_grid"] = {str(k): round(v, 2) for k, v in per_grid.items()}
        del bufs
        probe = res

    base = base1 = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(w, args.cpu_seconds, args.score)
        base1 = cpu_baseline(w, args.cpu_seconds / 2, args.score, threads=1) if host_cores() > 1 else base
    # counters were taken on the default step of the named workload only
    profiled = profiled_traffic(w.name) if args.score == "attn" and not args.budget else None
    line = {
        "metric": ("decode steps/s (full-cache attention step over the batch of one layer, no eviction)"
                   if args.score == "none" else
                   "decode steps/s (one fused attention+score+evict step over the batch of one layer)"),
        "value": round(steps_per_s, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": ("synthetic (seeded N(0,1) q/k/v, bf16 round-to-nearest-even)" if w.dtype == "bf16" else
                 "synthetic (seeded N(0,1) q/k/v, float32)"),
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "n_q_heads": w.n_q_heads,
            "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim,
            "budget": [int(bud.min()), int(bud.max())] if not w.fixed_budget else int(bud[0]),
            "sink": w.sink,
            "recent": w.recent,
            "score": args.score,
            "layer_caches": L,
            "launch": "eager" if args.eager else "hip-graph",
            "chunk_slots": chunk_slots,
            **({"initial_cache": "full-length prefills compressed to the budgets by lf_prefill_compress"}
               if w.prefill == "ragged" else {}),
        },
        "kv_GBps": round(achieved, 1),
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": profiled,
            "bytes_per_launch": step_bytes,
            "kernel": "lf_step_kernel",
        },
        "cpu_baseline": base,
        "cpu_baseline_1thread": base1,
        "wall_s_timed": round(wall, 4),
    }
    if probe:
        line["hbm_probe"] = probe
    if others:
        line["workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
