"""GPU tests of the HBM probes the benchmark uses as its bandwidth ceiling and
counter calibration: the copy reproduces its input exactly and the read
probe's checksum equals the XOR of the data."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from kv_cache_eviction_lf_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (1 << 22) + 48])
def test_probe_copy_and_read(nbytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = host.cuda()
    dst = torch.zeros_like(src)
    sink = torch.zeros(_lib.lf_probe_read_sink_words(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _lib.lf_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream)
    _lib.lf_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)
    words = host.numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_probe_empty_launch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    stream = torch.cuda.current_stream().cuda_stream
    for n in (1, 256, 4096):
        _lib.lf_probe_empty(n, stream)
    torch.cuda.synchronize()
    with pytest.raises(_lib.LFError):
        _lib.lf_probe_empty(0, stream)


@pytest.mark.parametrize("grid", [1, 256, 2048])
def test_probe_read_grid(grid):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nbytes = (1 << 20) + 32
    g = torch.Generator().manual_seed(grid)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = host.cuda()
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _lib.lf_probe_read_grid(src.data_ptr(), nbytes, grid, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want
    for bad in (0, _lib.lf_probe_read_sink_words() + 1):
        with pytest.raises(_lib.LFError):
            _lib.lf_probe_read_grid(src.data_ptr(), nbytes, bad, sink.data_ptr(), stream)
