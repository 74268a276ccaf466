"""Put generated workloads into device memory (torch tensors).

Plumbing only: draws come from workloads.generate and are copied unchanged
(bf16 values are exactly representable, so the cast is exact)."""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .configs import Workload
from .generate import budgets, initial_sequence, step_inputs


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def device_cache(w: Workload, device, threads: int = 8, max_budget: int | None = None):
    """Static cache tensors K, V [B][Hkv][max_budget][d] filled with every
    sequence's initial contents, plus seq_len (int64 [B]) and budgets (int32 [B])."""
    bud = budgets(w)
    S = int(bud.max()) if max_budget is None else int(max_budget)
    dt = torch_dtype(w)
    K = torch.zeros((w.batch, w.n_kv_heads, S, w.head_dim), dtype=dt, device=device)
    V = torch.zeros_like(K)
    seq_len = np.zeros(w.batch, dtype=np.int64)

    def fill(b):
        k, v, _, t = initial_sequence(w, b)
        return b, k, v, t

    with ThreadPoolExecutor(max(1, threads)) as ex:
        for b, k, v, t in ex.map(fill, range(w.batch)):
            n = k.shape[1]
            K[b, :, :n].copy_(torch.from_numpy(k).to(dt))
            V[b, :, :n].copy_(torch.from_numpy(v).to(dt))
            seq_len[b] = t
    return K, V, seq_len, bud


def device_step(w: Workload, step: int, device):
    """Inputs of one decode step for the whole batch: (q, k_new, v_new) device
    tensors, and the float32 host arrays they were made from."""
    q, k, v = step_inputs(w, step)
    dt = torch_dtype(w)
    dev = tuple(torch.from_numpy(x).to(dt).to(device) for x in (q, k, v))
    return dev, (q, k, v)


def device_step_pool(w: Workload, n: int, device, first_step: int = 0):
    """Inputs of ``n`` consecutive decode steps (from ``first_step``) drawn on the
    device, for timing runs that give every step fresh inputs: a list of
    (q, k_new, v_new) tensors.  Same distributions and structure as
    step_inputs (N(0,1) draws rounded to the workload's dtype, the key outlier
    channels scaled, anchor queries on event steps), from a seeded torch
    generator instead of the per-step numpy streams, so the values differ from
    step_inputs'."""
    from .generate import anchor_directions, anchor_event, outlier_channels

    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([w.seed, 0x5EED]).generate_state(1)[0]))
    dt = torch_dtype(w)
    ch = torch.as_tensor(outlier_channels(w), device=device)
    z = None
    if w.anchors:
        z = torch.as_tensor(np.stack([anchor_directions(w, b) for b in range(w.batch)]), dtype=torch.float32,
                            device=device)  # [B][Hkv][anchors][d]
    pool = []
    for s in range(first_step, first_step + n):
        q = torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=gen, device=device)
        k = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=gen, device=device)
        v = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=gen, device=device)
        ev = anchor_event(w, s)
        if ev is not None:
            q = z[:, :, ev, :].repeat_interleave(w.group, dim=1) + 0.5 * q
        if ch.numel():
            k[..., ch] *= w.outlier_scale
        pool.append((q.to(dt), k.to(dt), v.to(dt)))
    return pool
