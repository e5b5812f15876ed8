"""The decode under HIP graph capture: the scales are device pointers and the
workspace is the caller's, so a captured decode replays without host work.
The graph is replayed several times, with eager work and synchronizations in
between, and every replay must equal the eager result bit for bit."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import workloads
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_captured_decode_replays_bit_exact(dot):
    w = workloads.make("tiny", batch=4, s_q=2, h_q=64, seq_len=[900, 64, 1, 333], seed=31)
    t = gu.device_inputs(w)
    p = mla.params_for(t["q"], t["kv"], t["bt"], causal=True, dot=dot)
    splits = mla.resolve_splits(p, 0, mla.cu_count())
    ws = torch.zeros(max(mla.workspace_size(p, splits), 16), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((4, 2, 64, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((4, 2, 64), dtype=torch.float32, device="cuda:0")
    kw = dict(num_splits=splits, dot=dot, causal=True, out=out, lse=lse, workspace=ws)
    mla.decode(t["q"], t["kv"], t["bt"], t["sl"], t["ks"], t["vs"], **kw)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mla.decode(t["q"], t["kv"], t["bt"], t["sl"], t["ks"], t["vs"], stream=s, **kw)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        # eager work between replays
        mla.decode(t["q"], t["kv"], t["bt"], t["sl"], t["ks"], t["vs"], **kw)
        torch.cuda.synchronize()
