"""gfx942's e4m3fnuz cache on gfx950.

The cache holds torch float8_e4m3fnuz codes at scale amax/240 (largest fnuz
value, ROCm/aiter PR #6199, Technical details); the oracle decodes them from
the fnuz bit fields. Each workload's amax element carries the +-240 codes
(0x7F / 0xFF, NaN in e4m3fn), and the unowned rows hold 0x80, fnuz's NaN.

The bf16-dot path reads the cache exactly; every case checks that the kernel
reads the +-240 codes as 240. 0x80, fnuz's NaN, reads as zero in both modes.
The fp8-dot path turns each landed tile's codes into the e4m3fn codes
of the same values (oracle.fp8.fnuz_as_e4m3fn, checked here bit for bit on
all 256 codes): exact from 2^-6 of the scale up to 240, rounded to nearest
even below. Its cases are held to the fp8 tolerances both against the oracle
reading the fnuz cache exactly and against the oracle on the transcoded
cache, dense and sparse; per-token scales refuse an fnuz cache (host check,
no launch).
"""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import workloads
import gpu_util as gu

pytestmark = pytest.mark.gpu


CASES = [
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 64, "seq_len": [300, 1], "seed": 121}),
    ("tiny", {"batch": 3, "s_q": 2, "h_q": 48, "seq_len": [130, 64, 2], "seed": 122}),
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 16, "d_rope": 0, "seq_len": [257, 90], "seed": 123}),
    ("sparse", {"batch": 2, "seq_len": 5000, "topk": 300, "seed": 124}),
]
_CACHE = {}


def _case(name, **kw):
    key = (name, tuple(sorted((k, str(v)) for k, v in kw.items())))
    if key not in _CACHE:
        w = workloads.make(name, encoding="e4m3fnuz", **kw)
        _CACHE[key] = (w, gu.OracleCache(w), gu.device_inputs(w))
    return _CACHE[key]


def _has_top_codes(w):
    c = w.kv_cache[..., :w.d_nope]
    return bool(((c == 0x7F) | (c == 0xFF)).any())


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("idx", range(len(CASES)))
def test_fnuz_parity_bf16_dots(idx, splits):
    name, kw = CASES[idx]
    w, oc, t = _case(name, **kw)
    assert t["kv"].dtype == torch.float8_e4m3fnuz and _has_top_codes(w)
    res = gu.check(w, oc, "bf16", num_splits=splits, t=t)
    print(f"fnuz {name}{kw} splits={splits}: {res}")


def test_fnuz_full_benchmark_shape_bf16_dots():
    w, oc, t = _case("metric")
    res = gu.check(w, oc, "bf16", t=t)
    print(f"fnuz metric: {res}")


def test_fnuz_nan_code_reads_as_zero():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=16, seq_len=[100, 80], encoding="e4m3fnuz", seed=125)
    page = int(w.block_table[0, 0])
    w.kv_cache[page, 5, 17] = 0x80            # a visible key of sequence 0
    t = gu.device_inputs(w)
    out, lse = gu.run(w, t, "bf16", num_splits=1)
    w.kv_cache[page, 5, 17] = 0x00            # the oracle at the same byte read as zero
    ref_o, ref_l = gu.oracle(w)
    gu.compare(out, lse, ref_o, ref_l, dot="bf16")


def _transcoded(w):
    """The workload with its nope bytes replaced by the e4m3fn codes the fp8-dot
    path reads (oracle.fp8.fnuz_as_e4m3fn), as an e4m3fn cache."""
    import copy
    from oracle import fp8
    w2 = copy.copy(w)
    kv = w.kv_cache.copy()
    kv[..., :w.d_nope] = fp8.fnuz_as_e4m3fn(kv[..., :w.d_nope])
    w2.kv_cache = kv
    w2.encoding = "e4m3fn"
    return w2


def test_fnuz_transcoding_is_bit_exact():
    from oracle import fp8
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(3)[:763].to("cuda:0")   # ragged tail
    out = mla.debug_fnuz_to_e4m3fn(codes).cpu().numpy()
    assert np.array_equal(out, fp8.fnuz_as_e4m3fn(codes.cpu().numpy()))


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("idx", range(len(CASES)))
def test_fnuz_parity_fp8_dots(idx, splits):
    name, kw = CASES[idx]
    w, oc, t = _case(name, **kw)
    assert t["kv"].dtype == torch.float8_e4m3fnuz and _has_top_codes(w)
    res = gu.check(w, oc, "fp8", num_splits=splits, t=t)
    # against the oracle on the cache as the fp8 path reads it
    out, lse = gu.run(w, t, "fp8", num_splits=splits)
    oc2 = gu.OracleCache(_transcoded(w))
    rq = oc2.exact if gu.kernel_query_exact(w, "fp8") else oc2.qprime
    res2 = gu.compare(out, lse, *oc2.exact, rq[1], "fp8", ref_out_rows=rq[0])
    print(f"fnuz fp8 dots {name}{kw} splits={splits}: vs exact fnuz {res}; vs the transcoded cache {res2}")


def test_fnuz_full_benchmark_shape_fp8_dots():
    w, oc, t = _case("metric")
    res = gu.check(w, oc, "fp8", t=t)
    print(f"fnuz metric fp8 dots: {res}")


def test_fnuz_nan_code_reads_as_zero_fp8_dots():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=16, seq_len=[100, 80], encoding="e4m3fnuz", seed=127)
    page = int(w.block_table[0, 0])
    w.kv_cache[page, 5, 17] = 0x80
    t = gu.device_inputs(w)
    out, lse = gu.run(w, t, "fp8", num_splits=1)
    w.kv_cache[page, 5, 17] = 0x00
    oc = gu.OracleCache(_transcoded(w))
    rq = oc.exact if gu.kernel_query_exact(w, "fp8") else oc.qprime
    gu.compare(out, lse, *oc.exact, rq[1], "fp8", ref_out_rows=rq[0])


def test_fnuz_full_sparse_configuration_fp8_dots():
    w, oc, t = _case("sparse")
    res = gu.check(w, oc, "fp8", t=t)
    print(f"fnuz sparse configuration fp8 dots: {res}")


def test_fnuz_cache_is_refused_with_per_token_scales():
    name, kw = CASES[0]
    w, oc, t = _case(name, **kw)
    assert t["kv"].dtype == torch.float8_e4m3fnuz
    ks = torch.full((w.kv_cache.shape[0], 64), w.k_scale, dtype=torch.float32, device="cuda:0")
    with pytest.raises(mla.MlaError) as e:
        mla.decode(t["q"], t["kv"], t["bt"], t["sl"], ks, ks.clone(), num_splits=1, dot="fp8", causal=w.causal,
                   per_token_scales=True)
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED
