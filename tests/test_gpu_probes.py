"""The measurement probes bench.py reports against: they run through the C ABI
and fill their sinks (timing itself is bench.py's job)."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_mfma_probe_runs_and_counts_its_flops(dot):
    blocks, iters = 512, 8
    sentinel = -12345.0
    sink = torch.full((blocks * 256,), sentinel, dtype=torch.float32, device="cuda:0")
    flop = mla.mfma_probe(dot, iters, blocks, sink)
    torch.cuda.synchronize()
    assert flop == blocks * 4 * iters * 4 * (131072 if dot == "fp8" else 32768)
    # every thread stores its sum (the operands are arbitrary bit patterns, so it may be NaN)
    assert not (sink == sentinel).any()


def test_stream_read_probe_runs():
    src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda:0")
    sink = torch.full((1 << 16,), -1.0, dtype=torch.float32, device="cuda:0")
    mla.stream_read(src, sink)
    torch.cuda.synchronize()
    assert np.isfinite(sink[:4096].cpu().numpy()).all()
