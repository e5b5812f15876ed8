"""The allocation-free decode (mla_fp8_decode_noalloc) against the decode with a
caller workspace (mla_fp8_decode) on the same inputs: the two run the same
kernels with the same split plan, so output and lse must agree bit for bit;
both are also held to the oracle's tolerances. Two calls in a row, the second
smaller, so that partials left in the shared scratch by the first call cannot
leak into the second."""


import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import workloads
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _both(w, t, dot, num_splits):
    dev = t["q"].device
    b, s_q, h_q, _ = t["q"].shape
    out = torch.full((b, s_q, h_q, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((b, s_q, h_q), float("nan"), dtype=torch.float32, device=dev)
    kw = dict(num_splits=num_splits, dot=dot, causal=w.causal, softmax_scale=w.softmax_scale or 0.0,
              indices=t["idx"])
    mla.decode_noalloc(t["q"], t["kv"], t["bt"], t["sl"], t["ks"], t["vs"], out, lse, **kw)
    torch.cuda.synchronize()
    ref_out, ref_lse = mla.decode(t["q"], t["kv"], t["bt"], t["sl"], t["ks"], t["vs"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs from mla_fp8_decode"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "lse differs from mla_fp8_decode"
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _against_oracle(w, out, lse, dot):
    oc = gu.OracleCache(w)
    ref_o, ref_l = oc.exact
    ref_q = oc.exact if gu.kernel_query_exact(w, dot) else oc.qprime
    return gu.compare(out, lse, ref_o, ref_l, ref_q[1], dot, ref_out_rows=ref_q[0])


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_noalloc_matches_decode_on_two_calls(dot):
    big = workloads.make("tiny", batch=8, s_q=2, h_q=64,
                         seq_len=[3000, 700, 64, 1, 2500, 1800, 129, 4096], seed=41)
    small = workloads.make("tiny", batch=2, s_q=1, h_q=16, seq_len=[333, 1000], seed=42)
    for w, splits in ((big, 0), (small, 3)):
        t = gu.device_inputs(w)
        p = mla.params_for(t["q"], t["kv"], t["bt"], causal=w.causal, dot=dot)
        resolved = mla.resolve_splits(p, splits, mla.cu_count())
        print(f"noalloc {dot}: batch={w.batch} s_q={w.s_q} h_q={w.h_q} splits={resolved} "
              f"scratch={mla.workspace_size(p, resolved)}", flush=True)
        assert resolved > 1 and 0 < mla.workspace_size(p, resolved) <= mla.MLA_NOALLOC_SCRATCH_BYTES
        out, lse = _both(w, t, dot, splits)
        print("  vs oracle:", _against_oracle(w, out, lse, dot), flush=True)


def test_noalloc_one_split_needs_no_scratch():
    w = workloads.make("tiny", batch=3, s_q=1, h_q=16, seq_len=[77, 256, 5], seed=43)
    t = gu.device_inputs(w)
    out, lse = _both(w, t, "fp8", 1)
    _against_oracle(w, out, lse, "fp8")


def test_noalloc_at_the_benchmark_shape():
    # 64 sequences x 2 tokens x 64 heads over 8196 keys: four automatic splits,
    # 33.7 MB of partials in the fixed scratch; bitwise equal to mla_fp8_decode
    w = workloads.make("metric")
    t = gu.device_inputs(w)
    print(f"noalloc metric shape: batch={w.batch} seq_len={int(w.seq_lens.max())}", flush=True)
    _both(w, t, "fp8", 0)


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    # host check before any launch: 1024 sequences x 128 rows at 4 splits need 539 MB
    w = workloads.make("tiny", batch=2, s_q=2, h_q=64, seq_len=[64, 64], seed=44)
    t = gu.device_inputs(w)
    p = mla.make_params(batch=1024, s_q=2, h_q=64, num_pages=t["kv"].shape[0], max_pages_per_seq=1)
    assert mla.workspace_size(p, 4) > mla.MLA_NOALLOC_SCRATCH_BYTES
    out = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    st = mla.lib().mla_fp8_decode_noalloc(
        mla.ctypes.byref(p), mla._ptr(t["q"]), mla._ptr(t["kv"]), mla._ptr(t["bt"]), mla._ptr(t["sl"]),
        mla._ptr(t["ks"]), mla._ptr(t["vs"]), 4, mla._ptr(out), mla._ptr(lse), None, None)
    assert st == mla.MLA_ERR_SCRATCH
    assert torch.count_nonzero(out) == 0 and torch.count_nonzero(lse) == 0
