"""Parity of the HIP decode with the float64 oracle on seeded inputs.

Small cases span several tiles, ragged tails, several split counts and the
degenerate cases (empty sequences, causal rows with no key, a sequence of one
token, ragged head counts). The five workload configurations and the
benchmark shape then run at their full sizes, in the launch configuration the
benchmark uses (auto splits), compared element by element with the oracle.
All slack and unused pages are 0xFF (NaN) bytes, so any stray read of them
would poison the output and fail the finiteness check.
"""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import workloads
import gpu_util as gu

pytestmark = pytest.mark.gpu

_ORACLES = {}


def _case(name, **kw):
    key = (name, tuple(sorted((k, str(v)) for k, v in kw.items())))
    if key not in _ORACLES:
        w = workloads.make(name, **kw)
        _ORACLES[key] = (w, gu.OracleCache(w), gu.device_inputs(w))
    return _ORACLES[key]


SMALL = [
    ("tiny", {}),
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 64, "seq_len": [300, 1], "seed": 21}),
    ("tiny", {"batch": 3, "s_q": 2, "h_q": 48, "seq_len": [130, 64, 2], "seed": 22}),   # 96 rows: 3 row blocks
    ("tiny", {"batch": 2, "s_q": 1, "h_q": 8, "seq_len": [200, 33], "seed": 23}),
    ("tiny", {"batch": 2, "s_q": 4, "h_q": 64, "seq_len": [700, 3], "seed": 24}),      # 256 rows: 2 row groups
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 16, "d_rope": 0, "seq_len": [257, 90], "seed": 25}),
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 64, "seq_len": [600, 450], "causal": False, "seed": 26}),
]


@pytest.mark.parametrize("dot", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 2, 3, 0])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_small_dense(idx, splits, dot):
    name, kw = SMALL[idx]
    w, oc, t = _case(name, **kw)
    res = gu.check(w, oc, dot, num_splits=splits, t=t)
    print(f"{name}{kw} splits={splits} dot={dot}: {res}")


MAXIMA = [
    # the largest s_q the library takes (a 1024-token causal chunk: 4096 rows, 32 row groups)
    ("tiny", {"batch": 1, "s_q": 1024, "h_q": 4, "seq_len": [1100], "seed": 27}),
    # the largest h_q (1024 heads of one token: 8 row groups, ragged 2-page sequence)
    ("tiny", {"batch": 2, "s_q": 1, "h_q": 1024, "seq_len": [90, 700], "seed": 28}),
]


@pytest.mark.parametrize("dot", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [3, 0])
@pytest.mark.parametrize("idx", range(len(MAXIMA)))
def test_maximum_query_tokens_and_heads(idx, splits, dot):
    name, kw = MAXIMA[idx]
    w, oc, t = _case(name, **kw)
    res = gu.check(w, oc, dot, num_splits=splits, t=t)
    print(f"{name}{kw} splits={splits} dot={dot}: {res}")


@pytest.mark.parametrize("dot", ["bf16", "fp8"])
def test_empty_and_degenerate_rows(dot):
    # sequence lengths 0 and 1 with s_q = 2 (causal): whole sequences and single
    # rows without any visible key
    w, oc, t = _case("tiny", batch=4, s_q=2, h_q=32, seq_len=[0, 1, 65, 0], seed=31)
    for splits in (1, 4):
        gu.check(w, oc, dot, num_splits=splits, t=t)
    ref_l = oc.exact[1]
    assert np.isneginf(ref_l[0]).all() and np.isneginf(ref_l[1, 0]).all() and np.isfinite(ref_l[1, 1]).all()


@pytest.mark.parametrize("dot", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_small_sparse(dot, splits):
    w, oc, t = _case("sparse", batch=2, seq_len=5000, topk=300, seed=41)
    idx = t["idx"].clone()
    idx[0, 0, 5] = -1
    idx[1, 1, 17] = 5000       # == seq_len: skipped
    idx[1, 0, 0] = -7
    w.indices = idx.cpu().numpy()
    t = dict(t, idx=idx)
    oc = gu.OracleCache(w)
    gu.check(w, oc, dot, num_splits=splits, t=t)


@pytest.mark.parametrize("dot", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 3])
def test_sparse_repeated_indices_count_twice(dot, splits):
    """A position named more than once in a token's index list is attended to
    once per entry (the oracle counts it twice); repeats inside one 64-entry
    tile, across tiles and across splits."""
    w, oc, t = _case("sparse", batch=2, seq_len=5000, topk=300, seed=42)
    idx = w.indices.copy()
    idx[0, 0, 11] = idx[0, 0, 10]              # same tile
    idx[0, 1, 200] = idx[0, 1, 3]              # another tile (and split)
    idx[1, 0, 5:9] = idx[1, 0, 4]              # one position four more times
    idx[1, 1, 299] = idx[1, 1, 0]
    w.indices = idx
    t = dict(t, idx=torch.from_numpy(idx).to("cuda:0"))
    res = gu.check(w, gu.OracleCache(w), dot, num_splits=splits, t=t)
    print(f"repeated indices dot={dot} splits={splits}: {res}")


def test_more_splits_than_pages_gives_empty_splits():
    w, oc, t = _case("tiny", batch=2, s_q=2, h_q=64, seq_len=[130, 5], seed=51)
    for dot in ("bf16", "fp8"):
        gu.check(w, oc, dot, num_splits=9, t=t)


def test_transposed_v_reads_match_byte_gather():
    """The V^T operand read with ds_read_b64_tr_b8 equals a plain byte gather."""
    w, oc, t = _case("tiny", batch=2, s_q=2, h_q=64, seq_len=[300, 77], seed=61)
    for dot, base in (("bf16", 0), ("fp8", mla.MLA_VARIANT_DV_SPLIT)):
        a = gu.run(w, t, dot, 2, variant=base)
        b = gu.run(w, t, dot, 2, variant=base | mla.MLA_VARIANT_GATHER_V)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_deterministic_repeat():
    w, oc, t = _case("tiny", batch=2, s_q=2, h_q=64, seq_len=[1000, 333], seed=71)
    for dot in ("bf16", "fp8"):
        a = gu.run(w, t, dot, 0)
        b = gu.run(w, t, dot, 0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_v_scale_linearity_and_k_scale():
    w, oc, t = _case("tiny", batch=1, s_q=2, h_q=32, seq_len=[200], seed=81)
    o1, l1 = gu.run(w, t, "bf16", 1)
    t2 = dict(t, vs=t["vs"] * 2.0)
    o2, l2 = gu.run(w, t2, "bf16", 1)
    assert np.array_equal(l1, l2)
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-2, atol=1e-6)


# ---- the five configurations and the benchmark shape, full size ----------------

FULL = [("tiny", "bf16"), ("tiny", "fp8"), ("mtp", "bf16"), ("mtp", "fp8"), ("varlen", "fp8"),
        ("large", "bf16"), ("large", "fp8"), ("sparse", "bf16"), ("sparse", "fp8"), ("metric", "fp8"),
        ("metric", "bf16"),
        ("sparse16", "bf16"), ("sparse16", "fp8"), ("prefill", "bf16"), ("prefill", "fp8"),
        ("sparse_b1", "fp8"), ("sparse_b8", "bf16"), ("sparse_b64", "fp8"), ("sparse_b64", "bf16")]


@pytest.mark.parametrize("name,dot", FULL)
def test_full_config(name, dot):
    w, oc, t = _case(name)
    res = gu.check(w, oc, dot, t=t)
    print(f"full {name} dot={dot}: {res}")


@pytest.mark.parametrize("case", [("tiny", {"batch": 2, "s_q": 2, "h_q": 64, "seq_len": [700, 3], "seed": 91}),
                                  ("tiny", {"batch": 3, "s_q": 2, "h_q": 48, "seq_len": [130, 64, 2], "seed": 92}),
                                  ("tiny", {"batch": 2, "s_q": 1, "h_q": 16, "d_rope": 0, "seq_len": [257, 90], "seed": 93}),
                                  ("sparse", {"batch": 2, "seq_len": 3000, "topk": 200, "seed": 94}),
                                  ("metric", {})])
def test_dv_split_kernel_matches_row_block_kernel(case):
    """fp8 dots: splitting P.V over the waves by dv (P^T exchanged through LDS)
    issues the same products in the same order as the row-block kernel, so the
    two agree bit for bit, for every split count."""
    name, kw = case
    w, oc, t = _case(name, **kw)
    for splits in (1, 3, 0):
        a = gu.run(w, t, "fp8", splits, variant=mla.MLA_VARIANT_DV_SPLIT)
        b = gu.run(w, t, "fp8", splits, variant=mla.MLA_VARIANT_ROWS)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), f"splits={splits}"


# ---- the 16K-token sparse prefill (ROCm/aiter PR #6199, Results) -------------------
# Full size on the GPU; the oracle on a sample of 384 tokens spread over the
# 16K (sparse tokens are independent: each its own index list, no causal mask).

_SP = {}


def _sparse_prefill():
    if not _SP:
        w = workloads.make("sparse_prefill")
        _SP["w"], _SP["t"] = w, gu.device_inputs(w)
    return _SP["w"], _SP["t"]


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_sparse_prefill_16k_tokens(dot):
    import copy
    w, t = _sparse_prefill()
    assert w.s_q == 16384 and w.topk == 2048
    out, lse = gu.run(w, t, dot)
    tok = np.arange(7, w.s_q, w.s_q // 384)[:384]
    ws = copy.copy(w)
    ws.s_q = len(tok)
    ws.q_bits = w.q_bits[:, tok]
    ws.indices = w.indices[:, tok]
    oc = gu.OracleCache(ws)
    ref_q = oc.exact if gu.kernel_query_exact(w, dot) else oc.qprime
    res = gu.compare(out[:, tok], lse[:, tok], *oc.exact, ref_q[1], dot, ref_out_rows=ref_q[0])
    print(f"sparse prefill 16K, {dot} dots, {len(tok)} sampled tokens: {res}")


# ---- FlashMLA PR #82's H800 accuracy report, at its shape -----------------------
# b=64, s_q=2, mean_sk=4096, h_q=64, causal, fp8 cache: the "varlen" workload
# (seq lens U{2048..6144}). The page's figures (another machine, another
# implementation) are context; printed beside ours for the report.

PAGE_H800 = {"out_cos_diff": 6.64e-4, "out_rmse": 1.78e-3, "out_amax_diff": 4.80e-2,
             "lse_cos_diff": 3.26e-11, "lse_rmse": 7.12e-5, "lse_amax_diff": 2.16e-4}


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_accuracy_report_at_the_h800_shape(dot):
    w, oc, t = _case("varlen")
    assert w.batch == 64 and w.s_q == 2 and w.h_q == 64 and 2048 <= w.seq_lens.min() and w.seq_lens.max() <= 6144
    out, lse = gu.run(w, t, dot)
    ref_o, ref_l = oc.exact                      # the plain oracle (bf16 query) for both tensors
    live = ~np.isneginf(ref_l)
    m = {}
    m.update(gu.page_metrics(out[live], ref_o[live], "out"))
    m.update(gu.page_metrics(lse[live], ref_l[live], "lse"))
    print(f"H800-shape accuracy, {dot} dots: " + ", ".join(f"{k} {v:.3g} (page {PAGE_H800[k]:.3g})"
                                                          for k, v in m.items()))
    if dot == "fp8":
        # the same figures against the oracle at the query the kernel multiplies
        # (Q', quantized per row): what is left is the kernel's own arithmetic
        q_o, q_l = oc.qprime
        mq = {}
        mq.update(gu.page_metrics(out[live], q_o[live], "out"))
        mq.update(gu.page_metrics(lse[live], q_l[live], "lse"))
        print("H800-shape accuracy, fp8 dots, against the oracle at Q': "
              + ", ".join(f"{k} {v:.3g} (page {PAGE_H800[k]:.3g})" for k, v in mq.items()))
        assert mq["lse_amax_diff"] < 1e-3
    assert m["out_cos_diff"] < 1e-2 and m["lse_cos_diff"] < 1e-6
