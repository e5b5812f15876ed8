"""The C ABI on the host: the library loads, exports every declared symbol, and
its host-side checks return the documented status codes (no GPU needed: every
call here returns before any HIP launch)."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

import fp8_kv_cache_paged_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not mla.library_available():
        import __graft_entry__
        __graft_entry__.build()
    return mla.lib()


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "mla_fp8.h")).read()
    return sorted(set(re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_fp8_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared_symbols()
    assert len(names) == 17
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (mla_fp8_\w+)", out))
    assert set(names) <= exported
    assert exported <= set(names), f"undeclared exports: {exported - set(names)}"
    for n in names:
        assert hasattr(L, n)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(mla.MlaParams) == 16 * 4


def good(**kw):
    base = dict(batch=2, s_q=2, h_q=64, num_pages=10, max_pages_per_seq=5, kv_dtype=torch.uint8)
    base.update(kw)
    return mla.make_params(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, mla.MLA_OK),
    ({"kv_dtype": torch.float8_e4m3fn}, mla.MLA_OK),
    ({"kv_dtype": torch.float8_e4m3fnuz}, mla.MLA_OK),                         # fp8 dots (the default), dense
    ({"kv_dtype": torch.float8_e4m3fnuz, "topk": 8, "d_rope": 0}, mla.MLA_OK),   # fp8 dots, sparse
    ({"kv_dtype": torch.float8_e4m3fnuz, "per_token_scales": True}, mla.MLA_ERR_UNSUPPORTED),
    ({"kv_dtype": torch.float8_e4m3fnuz, "dot": "bf16"}, mla.MLA_OK),           # decoded to bf16 in registers
    ({"kv_dtype": torch.float8_e4m3fnuz, "dot": "bf16", "per_token_scales": True}, mla.MLA_ERR_UNSUPPORTED),
    ({"kv_dtype": torch.float8_e5m2}, mla.MLA_ERR_UNSUPPORTED),
    ({"kv_dtype": torch.int8}, mla.MLA_ERR_UNSUPPORTED),
    ({"kv_dtype": torch.bfloat16}, mla.MLA_ERR_UNSUPPORTED),
    ({"kv_dtype": 42}, mla.MLA_ERR_DTYPE),
    ({"h_kv": 2}, mla.MLA_ERR_UNSUPPORTED),
    ({"d_nope": 256}, mla.MLA_ERR_UNSUPPORTED),
    ({"d_rope": 32}, mla.MLA_ERR_UNSUPPORTED),
    ({"d_rope": 0}, mla.MLA_OK),
    ({"dv": 256}, mla.MLA_ERR_UNSUPPORTED),
    ({"page_block": 32}, mla.MLA_ERR_UNSUPPORTED),
    ({"batch": 0}, mla.MLA_ERR_SHAPE),
    ({"s_q": 0}, mla.MLA_ERR_SHAPE),
    ({"s_q": 1025}, mla.MLA_ERR_SHAPE),
    ({"per_token_scales": True}, mla.MLA_OK),
    ({"per_token_scales": True, "dot": "bf16"}, mla.MLA_OK),
    ({"per_token_scales": True, "topk": 64}, mla.MLA_OK),
    ({"s_q": 256}, mla.MLA_OK),
    ({"h_q": 0}, mla.MLA_ERR_SHAPE),
    ({"num_pages": 0}, mla.MLA_ERR_SHAPE),
    ({"max_pages_per_seq": 0}, mla.MLA_ERR_SHAPE),
    ({"topk": -1}, mla.MLA_ERR_SHAPE),
    ({"softmax_scale": float("nan")}, mla.MLA_ERR_SHAPE),
    ({"softmax_scale": float("inf")}, mla.MLA_ERR_SHAPE),
    ({"softmax_scale": -1.0}, mla.MLA_OK),
])
def test_validation_codes(L, kw, status):
    assert mla.validate(good(**kw)) == status


def test_validate_null_params(L):
    assert L.mla_fp8_validate(None) == mla.MLA_ERR_NULL


def test_status_strings(L):
    for s in range(9):
        assert mla.status_string(s) != "unknown status"
    assert mla.status_string(99) == "unknown status"


@pytest.mark.parametrize("batch,pages,expect", [(64, 129, 4), (32, 129, 8), (128, 129, 2), (256, 129, 1),
                                                (1, 129, 16), (3, 129, 16), (300, 129, 1), (32, 5, 5),
                                                (1, 1, 1)])
def test_auto_splits(L, batch, pages, expect, monkeypatch):
    # smallest s with batch * s >= 256 CUs, capped at 16 and at the pages per stream
    monkeypatch.delenv("MLA_FP8_NUM_SPLITS", raising=False)
    p = good(batch=batch, max_pages_per_seq=pages)
    assert mla.resolve_splits(p, 0, 256) == expect


def test_auto_splits_sparse_counts_tokens_as_groups(L, monkeypatch):
    monkeypatch.delenv("MLA_FP8_NUM_SPLITS", raising=False)
    p = good(batch=16, h_q=16, topk=2048, d_rope=0)
    assert mla.resolve_splits(p, 0, 256) == 8          # 32 (sequence, token) streams


def test_auto_splits_count_row_groups(L, monkeypatch):
    # a prefill chunk: 2 sequences x 256 tokens x 16 heads = 32 groups of 128
    # rows per sequence, so 64 workgroups per split and 4 splits fill 256 CUs
    monkeypatch.delenv("MLA_FP8_NUM_SPLITS", raising=False)
    p = good(batch=2, s_q=256, h_q=16, max_pages_per_seq=64)
    assert mla.resolve_splits(p, 0, 256) == 4
    q = good(batch=1, s_q=1024, h_q=64, max_pages_per_seq=64)   # 512 row groups: no split
    assert mla.resolve_splits(q, 0, 256) == 1


def test_explicit_and_env_splits(L, monkeypatch):
    p = good(max_pages_per_seq=200)
    assert mla.resolve_splits(p, 3, 256) == 3
    assert mla.resolve_splits(p, 1000, 256) == mla.MLA_MAX_SPLITS
    assert mla.resolve_splits(p, -1, 256) < 0
    monkeypatch.setenv("MLA_FP8_NUM_SPLITS", "7")
    assert mla.resolve_splits(p, 0, 256) == 7
    assert mla.resolve_splits(p, 2, 256) == 2
    assert mla.resolve_splits(good(batch=0), 0, 256) == -mla.MLA_ERR_SHAPE


def test_workspace_size(L):
    p = good(batch=64, s_q=2, h_q=64)
    assert mla.workspace_size(p, 1) == 0
    frags = 4 * 64 * 4
    assert mla.workspace_size(p, 4) == frags * (16 * 64 * 16 * 2 + 32 * 4)
    q = good(batch=3, s_q=1, h_q=16)                  # one row block per sequence
    assert mla.workspace_size(q, 2) == 2 * 3 * (16 * 64 * 16 * 2 + 32 * 4)
    assert mla.workspace_size(good(batch=0), 4) == 0
    # per-token scales: one more f32 per partial row (its value scale)
    pt = good(batch=64, s_q=2, h_q=64, per_token_scales=True)
    assert mla.workspace_size(pt, 4) == frags * (16 * 64 * 16 * 2 + 2 * 32 * 4)


def _decode_call(L, p, **ptrs):
    d = dict(q=16, kv=16, bt=16, sl=16, ks=16, vs=16, out=16, lse=16, idx=None, ws=None)
    d.update(ptrs)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.mla_fp8_decode(ctypes.byref(p), v(d["q"]), v(d["kv"]), v(d["bt"]), v(d["sl"]), v(d["ks"]),
                            v(d["vs"]), 1, v(d["out"]), v(d["lse"]), v(d["idx"]), v(d["ws"]), 0, None)


def test_decode_rejects_before_any_launch(L):
    # host pointers that are never dereferenced: every call fails a host check first
    p = good()
    assert _decode_call(L, p, q=None) == mla.MLA_ERR_NULL
    assert _decode_call(L, p, ks=None) == mla.MLA_ERR_NULL      # fp8 cache without scales
    assert _decode_call(L, p, vs=None) == mla.MLA_ERR_NULL
    assert _decode_call(L, p, lse=None) == mla.MLA_ERR_NULL
    assert _decode_call(L, good(topk=8), idx=None) == mla.MLA_ERR_NULL
    assert _decode_call(L, p, q=24) == mla.MLA_ERR_ALIGN
    assert _decode_call(L, p, kv=8) == mla.MLA_ERR_ALIGN
    assert _decode_call(L, p, sl=18) == mla.MLA_ERR_ALIGN
    assert _decode_call(L, good(kv_dtype=torch.float8_e5m2)) == mla.MLA_ERR_UNSUPPORTED
    # explicit splits > 1 need a workspace
    st = L.mla_fp8_decode(ctypes.byref(p), *[ctypes.c_void_p(16)] * 6, 2, ctypes.c_void_p(16),
                          ctypes.c_void_p(16), None, None, 0, None)
    assert st == mla.MLA_ERR_WORKSPACE


def test_noalloc_rejects_before_any_launch(L):
    # host pointers that are never dereferenced; explicit split counts, so no HIP call
    v = ctypes.c_void_p
    p = good(batch=1024, s_q=2, h_q=64)
    assert mla.workspace_size(p, 4) > mla.MLA_NOALLOC_SCRATCH_BYTES
    args = [ctypes.byref(p)] + [v(16)] * 6
    assert L.mla_fp8_decode_noalloc(*args, 4, v(16), v(16), None, None) == mla.MLA_ERR_SCRATCH
    assert L.mla_fp8_decode_noalloc(*args, 4, None, v(16), None, None) == mla.MLA_ERR_NULL
    assert L.mla_fp8_decode_noalloc(*args, 4, v(24), v(16), None, None) == mla.MLA_ERR_ALIGN
    bad = good(h_kv=2)
    assert L.mla_fp8_decode_noalloc(ctypes.byref(bad), *[v(16)] * 6, 4, v(16), v(16), None,
                                    None) == mla.MLA_ERR_UNSUPPORTED


def test_decode_variant_rejects_unknown_bits_before_any_launch(L):
    p = good()
    args = [ctypes.byref(p)] + [ctypes.c_void_p(16)] * 6 + [1, ctypes.c_void_p(16), ctypes.c_void_p(16), None,
                                                             None, 0]
    assert L.mla_fp8_debug_decode_variant(*args, 8, None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_debug_decode_variant(*args, -1, None) == mla.MLA_ERR_SHAPE
    # known bits pass the variant check and fail later on the invalid params
    bad = good(h_kv=2)
    args[0] = ctypes.byref(bad)
    assert L.mla_fp8_debug_decode_variant(*args, mla.MLA_VARIANT_ROWS, None) == mla.MLA_ERR_UNSUPPORTED
    # an fnuz cache with fp8 dots has no variant kernels
    fz = good(kv_dtype=torch.float8_e4m3fnuz)
    args[0] = ctypes.byref(fz)
    assert L.mla_fp8_debug_decode_variant(*args, mla.MLA_VARIANT_ROWS, None) == mla.MLA_ERR_UNSUPPORTED


def test_debug_exports_check_arguments(L):
    assert L.mla_fp8_debug_fnuz_to_e4m3fn(None, ctypes.c_void_p(16), 4, None) == mla.MLA_ERR_NULL
    assert L.mla_fp8_debug_fnuz_to_e4m3fn(ctypes.c_void_p(16), ctypes.c_void_p(16), -1, None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_debug_decode_e4m3fn(None, None, None, 4, None) == mla.MLA_ERR_NULL
    assert L.mla_fp8_debug_quantize_q(ctypes.c_void_p(16), 1, 100, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                      None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_bench_stream_read(ctypes.c_void_p(16), 17, ctypes.c_void_p(16), None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_debug_gather(ctypes.byref(good(h_kv=3)), None, None, None, None, None) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_fp8_debug_gather_ws(ctypes.byref(good(h_kv=3)), None, None, None, None, None) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_fp8_debug_gather_ws(ctypes.byref(good()), None, None, None, None, None) == mla.MLA_ERR_NULL


# ---- quantize-on-write: host checks (every call returns before a launch) ----

def _q(L, n=4, d_rope=64, pages=2, ckv=16, rope=16, slots=16, kv=16, ks=16, vs=16, cs=1, ws=16,
       ws_bytes=None):
    vp = ctypes.c_void_p
    wsb = L.mla_fp8_quantize_kv_workspace_size() if ws_bytes is None else ws_bytes
    return L.mla_fp8_quantize_kv(n, d_rope, pages, vp(ckv) if ckv else None, vp(rope) if rope else None,
                                 vp(slots) if slots else None, vp(kv) if kv else None, vp(ks) if ks else None,
                                 vp(vs) if vs else None, cs, vp(ws) if ws else None, wsb, None)


def test_quantize_workspace_size(L):
    assert L.mla_fp8_quantize_kv_workspace_size() == 4096


@pytest.mark.parametrize("kw,status", [
    ({"n": -1}, mla.MLA_ERR_SHAPE),
    ({"pages": 0}, mla.MLA_ERR_SHAPE),
    ({"cs": 3}, mla.MLA_ERR_SHAPE),
    ({"n": 0, "cs": 2, "ws": 0}, mla.MLA_OK),                     # per token, nothing to write
    ({"d_rope": 32}, mla.MLA_ERR_UNSUPPORTED),
    ({"ks": 0}, mla.MLA_ERR_NULL),
    ({"vs": 0}, mla.MLA_ERR_NULL),
    ({"kv": 0}, mla.MLA_ERR_NULL),
    ({"ckv": 0}, mla.MLA_ERR_NULL),
    ({"slots": 0}, mla.MLA_ERR_NULL),
    ({"rope": 0}, mla.MLA_ERR_NULL),
    ({"ws": 0}, mla.MLA_ERR_WORKSPACE),
    ({"ws_bytes": 4000}, mla.MLA_ERR_WORKSPACE),
    ({"ckv": 8}, mla.MLA_ERR_ALIGN),
    ({"kv": 24}, mla.MLA_ERR_ALIGN),
    ({"ks": 2}, mla.MLA_ERR_ALIGN),
    ({"n": 0, "cs": 0}, mla.MLA_OK),                              # nothing to do: no launch
    ({"n": 0, "cs": 0, "ckv": 0, "slots": 0, "rope": 0}, mla.MLA_OK),
])
def test_quantize_host_checks(L, kw, status):
    assert _q(L, **kw) == status


def test_mfma_probe_rejects_before_any_launch(L):
    # host checks only: none of these reaches a kernel launch
    assert L.mla_fp8_bench_mfma(mla.MLA_DOT_FP8, 4, 4, None, None) == mla.MLA_ERR_NULL
    assert L.mla_fp8_bench_mfma(7, 4, 4, 256, None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_bench_mfma(mla.MLA_DOT_BF16, 0, 4, 256, None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_bench_mfma(mla.MLA_DOT_FP8, 4, 0, 256, None) == mla.MLA_ERR_SHAPE
    assert L.mla_fp8_bench_mfma(mla.MLA_DOT_FP8, 4, 4, 258, None) == mla.MLA_ERR_ALIGN
    with pytest.raises(ValueError):
        mla.mfma_probe("fp16", 4, 4, torch.empty(1024))
    with pytest.raises(ValueError):
        mla.mfma_probe("fp8", 4, 4, torch.empty(1024))   # host tensor
