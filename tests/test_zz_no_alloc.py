"""The allocation-free prefill compression (lf_prefill_compress_noalloc, its
scratch a static device array inside the library) against lf_prefill_compress
with a caller workspace, through the C ABI: kept positions and the copied K/V
rows must be identical, on two calls in a row, the second one smaller."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from kv_cache_eviction_lf_amd import _lib
from workloads import Workload, prefill_inputs

pytestmark = pytest.mark.gpu


def _run_both(w, budgets, prefill, max_prefill):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = prefill_inputs(w, max_prefill)
    qd, kd, vd = (torch.from_numpy(x).to(dev, tdt) for x in (q, k, v))
    max_budget = max(budgets)
    cfg = _lib.make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, max_budget, w.sink, w.recent,
                           _lib.LF_BF16 if w.dtype == "bf16" else _lib.LF_F32)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (False, True):
        kc = torch.full((w.batch, w.n_kv_heads, max_budget, w.head_dim), 7.0, dtype=tdt, device=dev)
        vc = torch.full_like(kc, -7.0)
        kept = torch.full((w.batch, w.n_kv_heads, max_budget), -5, dtype=torch.int32, device=dev)
        if noalloc:
            _lib.lf_prefill_compress_noalloc(cfg, budgets, prefill, max_prefill, qd.data_ptr(), kd.data_ptr(),
                                             vd.data_ptr(), kc.data_ptr(), vc.data_ptr(), kept.data_ptr(), stream)
        else:
            wb = _lib.lf_prefill_work_bytes(cfg, max_prefill)
            work = torch.empty(wb, dtype=torch.uint8, device=dev)
            _lib.lf_prefill_compress(cfg, budgets, prefill, max_prefill, qd.data_ptr(), kd.data_ptr(),
                                     vd.data_ptr(), kc.data_ptr(), vc.data_ptr(), kept.data_ptr(), work.data_ptr(),
                                     wb, stream)
        torch.cuda.synchronize()
        outs.append((kept.cpu(), kc.cpu(), vc.cpu()))
    (k0, kc0, vc0), (k1, kc1, vc1) = outs
    assert torch.equal(k0, k1), "kept positions differ"
    assert torch.equal(kc0.view(torch.int16) if tdt == torch.bfloat16 else kc0.view(torch.int32),
                       kc1.view(torch.int16) if tdt == torch.bfloat16 else kc1.view(torch.int32)), "K rows differ"
    assert torch.equal(vc0.view(torch.int16) if tdt == torch.bfloat16 else vc0.view(torch.int32),
                       vc1.view(torch.int16) if tdt == torch.bfloat16 else vc1.view(torch.int32)), "V rows differ"
    # the compression did run: every sequence keeps min(prefill, budget) increasing
    # positions, sinks and the recent window among them; slots past them are untouched
    for b in range(w.batch):
        nb, P = min(prefill[b], budgets[b]), prefill[b]
        got = k1[b, :, :nb].numpy()
        assert np.all(np.diff(got, axis=1) > 0) and np.all(k1[b, :, nb:].numpy() == -5)
        assert np.all(got[:, : w.sink] == np.arange(w.sink))
        assert np.all(got[:, nb - min(w.recent, nb):] == np.arange(P - min(w.recent, nb), P))
        assert torch.all(kc1[b, :, nb:] == 7.0)


def test_noalloc_matches_workspace_entry_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = Workload("noalloc_big", 4, 32, 8, 128, "bf16", 1024, 2048, 4, 64, 0, seed=41)
    print("[noalloc] call 1: B=4 Hq=32 Hkv=8 d=128 bf16 prefill up to 4096", flush=True)
    _run_both(big, [1024, 2048, 1500, 2048], [4096, 3000, 1500, 4000], 4096)
    small = Workload("noalloc_small", 2, 10, 2, 128, "f32", 200, 250, 4, 8, 0, seed=42)
    print("[noalloc] call 2: B=2 Hq=10 Hkv=2 d=128 f32 prefill up to 640", flush=True)
    _run_both(small, [200, 250], [600, 100], 640)
