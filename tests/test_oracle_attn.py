"""Pins of the oracle's attention, split form and query quantization (CPU only).

Each check here is independent of the oracle's own arithmetic: closed forms,
brute-force loops over torch-decoded bytes, special cases that reduce to a
plain softmax, and invariances that hold for any correct implementation.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import attn, fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _single_seq(nope_codes, rope_bits=None, q_bits=None, *, shuffle_seed=None):
    """A one-sequence paged cache holding the given rows (n keys)."""
    n, d_nope = nope_codes.shape
    d_rope = 0 if rope_bits is None else rope_bits.shape[1]
    pages = max(-(-n // 64), 1)
    order = np.arange(pages + 1)
    if shuffle_seed is not None:
        order = np.random.default_rng(shuffle_seed).permutation(pages + 1)
    cache = np.full((pages + 1, 64, d_nope + 2 * d_rope), 0xFF, dtype=np.uint8)
    bt = order[:pages].astype(np.int32)[None, :]
    for j in range(n):
        cache[bt[0, j // 64], j % 64, :d_nope] = nope_codes[j]
        if d_rope:
            cache[bt[0, j // 64], j % 64, d_nope:] = rope_bits[j].view(np.uint8)
    return cache, bt, np.array([n], dtype=np.int32)


def test_equal_logits_give_mean_of_v_and_log_count():
    """q = 0: every visible key scores 0, so out = mean(V) and lse = ln L."""
    w = workloads.make("tiny", batch=2, s_q=2, h_q=3, seq_len=[130, 1], causal=True)
    q = np.zeros_like(w.q_bits)
    out, lse = attn.mla_decode(q, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                               w.v_scale, d_rope=w.d_rope, causal=True)
    for b in range(2):
        sk = int(w.seq_lens[b])
        for i in range(2):
            L = sk - (1 - i)
            if L <= 0:
                assert np.all(out[b, i] == 0) and np.all(np.isneginf(lse[b, i]))
                continue
            pos = np.arange(L)
            rows = w.kv_cache[w.block_table[b, pos // 64], pos % 64, :512]
            mean_v = _torch_decode(rows).mean(axis=0) * w.v_scale
            np.testing.assert_allclose(out[b, i], np.broadcast_to(mean_v, out[b, i].shape),
                                       rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(lse[b, i], math.log(L), rtol=0, atol=1e-12)


def test_one_dominant_key_gives_its_value_row():
    n, d = 200, 512
    codes = np.zeros((n, d), dtype=np.uint8)
    dom = 137
    codes[dom, :] = 0x38                        # 1.0 everywhere
    codes[:, 5] = 0x40                          # a shared coordinate (2.0) on every key
    rope = np.zeros((n, 64), dtype=np.uint16)
    cache, bt, sl = _single_seq(codes, rope, shuffle_seed=1)
    q = np.zeros((1, 1, 2, 576), dtype=np.uint16)
    q[..., :512] = fp8.f32_to_bf16_bits(np.float32(4.0))
    out, lse = attn.mla_decode(q, cache, bt, sl, 1.0, 0.5, causal=False, softmax_scale=1 / 24)
    z_dom = (4.0 * 511 * 1.0 + 4.0 * 2.0) / 24  # 511 ones and the shared coordinate's 2.0
    z_other = 4.0 * 2.0 / 24
    assert z_dom - z_other > 60
    v_dom = _torch_decode(codes[dom]) * 0.5
    np.testing.assert_allclose(out[0, 0, 0], v_dom, rtol=1e-14, atol=1e-20)
    np.testing.assert_allclose(lse[0, 0, 0], z_dom, rtol=0, atol=1e-12)


def test_softmax_tail_fixture():
    """One key at logit 9, 2047 keys at logit 0 (the aiter page's tail test)."""
    with open(os.path.join(GOLDEN, "softmax_tail.json")) as f:
        g = json.load(f)
    n = g["tail_keys"] + 1
    codes = np.zeros((n, 512), dtype=np.uint8)
    codes[0, 0] = 0x49                          # 4.5 on a coordinate only the first key has
    codes[1:, 1] = 0x38                         # the tail's value: 1.0 in dim 1
    codes[0, 2] = 0x38                          # the dominant key's value: 1.0 in dim 2
    cache, bt, sl = _single_seq(codes, shuffle_seed=2)
    q = np.zeros((1, 1, 1, 512), dtype=np.uint16)
    q[..., 0] = fp8.f32_to_bf16_bits(np.float32(2.0))   # 2.0 * 4.5 = 9 exactly
    out, lse = attn.mla_decode(q, cache, bt, sl, 1.0, 1.0, d_rope=0, causal=False,
                               softmax_scale=1.0)
    gap = g["dominant_logit"] - g["tail_logit"]
    tail = g["tail_keys"] * math.exp(-gap)
    share = tail / (1 + tail)
    assert abs(share - 0.20167) < 1e-5
    assert abs(share - g["page_tail_share_approx"]) < 0.01
    np.testing.assert_allclose(out[0, 0, 0, 1], share, rtol=1e-13)
    np.testing.assert_allclose(out[0, 0, 0, 2], 1 - share, rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0, 0], 9 + math.log1p(tail), rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - 9.22524) < 1e-5


def _brute_force(q_bits, cache, bt, seq_lens, ks, vs, d_nope, d_rope, causal, scale,
                 indices=None):
    """Scalar loops over torch-decoded bytes: one row at a time, one key at a time."""
    b, s_q, h_q, d = q_bits.shape
    q = _torch_bf16(q_bits)
    out = np.zeros((b, s_q, h_q, d_nope))
    lse = np.full((b, s_q, h_q), -math.inf)
    for bi in range(b):
        sk = int(seq_lens[bi])
        for i in range(s_q):
            if indices is not None:
                keys = [int(j) for j in indices[bi, i] if 0 <= j < sk]
            else:
                keys = list(range(sk - (s_q - 1 - i) if causal else sk))
            for h in range(h_q):
                zs, vrows = [], []
                for j in keys:
                    row = cache[bt[bi, j // 64], j % 64]
                    # per-tensor scales, or per-token arrays [pages, 64]
                    kss = float(ks[bt[bi, j // 64], j % 64]) if np.ndim(ks) else ks
                    vss = float(vs[bt[bi, j // 64], j % 64]) if np.ndim(vs) else vs
                    kn = _torch_decode(row[:d_nope])
                    kr = _torch_bf16(row[d_nope:].view(np.uint16)) if d_rope else np.zeros(0)
                    s = 0.0
                    for t in range(d_nope):
                        s += q[bi, i, h, t] * kn[t] * kss
                    for t in range(d_rope):
                        s += q[bi, i, h, d_nope + t] * kr[t]
                    zs.append(scale * s)
                    vrows.append(kn * vss)
                if not zs:
                    continue
                m = max(zs)
                ws = [math.exp(z - m) for z in zs]
                l = sum(ws)
                acc = np.zeros(d_nope)
                for wgt, v in zip(ws, vrows):
                    acc += wgt * v
                out[bi, i, h] = acc / l
                lse[bi, i, h] = m + math.log(l)
    return out, lse


@pytest.mark.parametrize("seq_lens,causal", [([70, 1], True), ([0, 65], False), ([129, 2], True)])
def test_brute_force_dense(seq_lens, causal):
    w = workloads.make("tiny", batch=2, s_q=2, h_q=2, seq_len=seq_lens, causal=causal, seed=11)
    out, lse = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                               w.v_scale, causal=causal)
    ref_o, ref_l = _brute_force(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                                w.v_scale, 512, 64, causal, 1 / 24)
    np.testing.assert_allclose(out, ref_o, rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_l))
    f = np.isfinite(ref_l)
    np.testing.assert_allclose(lse[f], ref_l[f], rtol=0, atol=1e-11)


def test_brute_force_sparse_with_invalid_entries():
    w = workloads.make("sparse", batch=2, s_q=2, h_q=2, seq_len=300, topk=40, seed=12)
    idx = w.indices.copy()
    idx[0, 0, 3] = -1
    idx[1, 1, 7] = 300          # == seq_len: skipped
    idx[1, 0, 9] = idx[1, 0, 10]  # a repeated entry counts twice
    out, lse = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                               w.v_scale, d_rope=0, causal=False, indices=idx)
    ref_o, ref_l = _brute_force(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                                w.v_scale, 512, 0, False, 1 / math.sqrt(512), indices=idx)
    np.testing.assert_allclose(out, ref_o, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-11)


def test_sparse_over_all_positions_equals_dense():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=4, seq_len=[200, 77], causal=False, seed=5)
    idx = np.full((2, 2, 256), -1, dtype=np.int32)
    for b in range(2):
        for i in range(2):
            idx[b, i, :w.seq_lens[b]] = np.random.default_rng(b * 2 + i).permutation(w.seq_lens[b])
    d_o, d_l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                               w.v_scale, causal=False)
    s_o, s_l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                               w.v_scale, causal=False, indices=idx)
    np.testing.assert_allclose(s_o, d_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s_l, d_l, rtol=0, atol=1e-12)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 5, 8])
def test_split_invariance_dense(num_splits):
    w = workloads.make("tiny", batch=3, s_q=2, h_q=4, seq_len=[300, 65, 1], causal=True, seed=9)
    ref_o, ref_l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens,
                                   w.k_scale, w.v_scale, causal=True)
    po, pl = attn.split_partials(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                                 w.v_scale, num_splits, causal=True)
    o, l = attn.combine(po, pl)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.isneginf(l), np.isneginf(ref_l))
    f = np.isfinite(ref_l)
    np.testing.assert_allclose(l[f], ref_l[f], rtol=0, atol=1e-12)
    if num_splits >= 2:
        # sequence 2 has one page: all but one split are empty for it
        assert np.isneginf(pl[:, 2]).sum() >= (num_splits - 1) * 2 * 4


@pytest.mark.parametrize("num_splits", [1, 4, 7])
def test_split_invariance_sparse(num_splits):
    w = workloads.make("sparse", batch=2, s_q=2, h_q=3, seq_len=1000, topk=300, seed=4)
    ref_o, ref_l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens,
                                   w.k_scale, w.v_scale, d_rope=0, causal=False, indices=w.indices)
    po, pl = attn.split_partials(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                                 w.v_scale, num_splits, d_rope=0, causal=False, indices=w.indices)
    o, l = attn.combine(po, pl)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


def test_combine_all_empty_gives_zero_and_neg_inf():
    o = np.random.default_rng(0).standard_normal((3, 2, 5))
    l = np.full((3, 2), -np.inf)
    out, lse = attn.combine(o, l)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_block_table_relabelling_invariance():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=3, seq_len=[190, 64], causal=True, seed=3)
    o1, l1 = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                             w.v_scale, causal=True)
    perm = np.random.default_rng(1).permutation(w.kv_cache.shape[0])
    cache2 = np.empty_like(w.kv_cache)
    cache2[perm] = w.kv_cache
    bt2 = perm[w.block_table].astype(np.int32)
    o2, l2 = attn.mla_decode(w.q_bits, cache2, bt2, w.seq_lens, w.k_scale, w.v_scale, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_v_scale_is_linear_and_k_scale_spares_rope():
    w = workloads.make("tiny", batch=1, s_q=1, h_q=4, seq_len=100, seed=8)
    args = (w.q_bits, w.kv_cache, w.block_table, w.seq_lens)
    o1, l1 = attn.mla_decode(*args, w.k_scale, w.v_scale)
    o2, l2 = attn.mla_decode(*args, w.k_scale, 2.5 * w.v_scale)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(l1, l2)
    # with the nope part of q zeroed, k_scale cannot matter: rope is unscaled
    q0 = w.q_bits.copy()
    q0[..., :512] = 0
    o3, l3 = attn.mla_decode(q0, *args[1:], w.k_scale, w.v_scale)
    o4, l4 = attn.mla_decode(q0, *args[1:], 7.0 * w.k_scale, w.v_scale)
    np.testing.assert_array_equal(o3, o4)
    np.testing.assert_array_equal(l3, l4)


def test_causal_rows_see_bottom_right_aligned_prefixes():
    w = workloads.make("tiny", batch=1, s_q=2, h_q=2, seq_len=150, causal=True, seed=6)
    o1, l1 = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale,
                             w.v_scale, causal=True)
    cache2 = w.kv_cache.copy()
    last = 149
    cache2[w.block_table[0, last // 64], last % 64, :512] = 0x38
    o2, l2 = attn.mla_decode(w.q_bits, cache2, w.block_table, w.seq_lens, w.k_scale,
                             w.v_scale, causal=True)
    np.testing.assert_array_equal(o1[0, 0], o2[0, 0])   # token 0 sees keys 0..148
    assert np.any(o1[0, 1] != o2[0, 1])                 # token 1 sees key 149 too


def test_q_row_exponent_is_the_smallest_power_of_two():
    rng = np.random.default_rng(1)
    vals = np.concatenate([np.abs(rng.standard_normal(2000)) * 10.0 ** rng.integers(-8, 8, 2000),
                           448.0 * 2.0 ** np.arange(-20, 20), [1e-30, 447.99, 448.0, 448.01]])
    for a in vals:
        e = attn.q_row_exponent(float(a))
        assert a <= 448 * 2.0 ** e
        assert a > 448 * 2.0 ** (e - 1)
    assert attn.q_row_exponent(0.0) == 0


def test_quantize_q_rows_against_torch_cast():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=8, seq_len=64, seed=2)
    qn = fp8.bf16_bits_to_f64(w.q_bits)[..., :512]
    qn[0, 0, 0] = 0.0
    qn[1, 1, 3] *= 1e-3
    codes, exps = attn.quantize_q_rows(qn)
    assert exps[0, 0, 0] == 0 and np.all(codes[0, 0, 0] == 0)
    scaled = (qn * np.ldexp(1.0, -exps.astype(np.int64))[..., None]).astype(np.float32)
    ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    amax = np.abs(scaled).max(axis=-1)
    assert np.all(amax[exps != 0] > 224) and np.all(amax <= 448)


# ---- per-token scales ([pages, 64], one k and one v scale per cache row) ----

def _per_token_scales(w, seed, spread=8.0):
    rng = np.random.default_rng(seed)
    shape = (w.kv_cache.shape[0], 64)
    ks = (w.k_scale * rng.uniform(1.0 / spread, 1.0, shape)).astype(np.float32)
    vs = (w.v_scale * rng.uniform(1.0 / spread, 1.0, shape)).astype(np.float32)
    return ks, vs


def test_per_token_scales_brute_force():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=2, seq_len=[150, 70], seed=41)
    ks, vs = _per_token_scales(w, 42)
    out, lse = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, causal=True)
    ref_o, ref_l = _brute_force(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, 512, 64, True, 1 / 24)
    np.testing.assert_allclose(out, ref_o, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-11)


def test_uniform_per_token_scales_equal_per_tensor():
    w = workloads.make("tiny", batch=2, s_q=2, h_q=4, seq_len=[300, 5], seed=43)
    shape = (w.kv_cache.shape[0], 64)
    ks = np.full(shape, w.k_scale, dtype=np.float64)
    vs = np.full(shape, w.v_scale, dtype=np.float64)
    a = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, causal=True)
    b = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale, w.v_scale, causal=True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_per_token_v_scales_are_linear_and_unused_rows_do_not_matter():
    w = workloads.make("tiny", batch=1, s_q=2, h_q=4, seq_len=[130], seed=44)
    ks, vs = _per_token_scales(w, 45)
    o1, l1 = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, causal=True)
    o2, l2 = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, 2 * vs, causal=True)
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-13, atol=0)
    np.testing.assert_array_equal(l1, l2)
    # scales of rows no sequence uses (slack of the last page, unused pages)
    used = np.zeros(ks.shape, dtype=bool)
    pos = np.arange(130)
    used[w.block_table[0, pos // 64], pos % 64] = True
    ks3, vs3 = ks.copy(), vs.copy()
    ks3[~used] = np.nan
    vs3[~used] = np.nan
    o3, l3 = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks3, vs3, causal=True)
    np.testing.assert_array_equal(o3, o1)
    np.testing.assert_array_equal(l3, l1)


@pytest.mark.parametrize("num_splits", [2, 3, 5])
def test_split_invariance_per_token(num_splits):
    w = workloads.make("tiny", batch=2, s_q=2, h_q=4, seq_len=[400, 65], seed=46)
    ks, vs = _per_token_scales(w, 47)
    o, l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, causal=True)
    po, pl = attn.split_partials(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, num_splits, causal=True)
    co, cl = attn.combine(po, pl)
    np.testing.assert_allclose(co, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cl, l, rtol=0, atol=1e-12)


# ---- Q' (the fp8-dot path's dequantized query) --------------------------------

def _brute_force_q_prime(q_row):
    """Q' of one row from the definition, with an outside codec: the smallest
    integer e with amax <= 448 * 2**e (searched upwards), torch's
    float8_e4m3fn cast of q * 2**-e, torch's decode, times 2**e."""
    amax = float(np.abs(q_row).max())
    e = 0
    if amax > 0:
        e = -200
        while amax > 448.0 * 2.0 ** e:
            e += 1
    scaled = torch.from_numpy(q_row * 2.0 ** -e)
    back = scaled.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return back * 2.0 ** e, e


def _e4m3fn_half_step(x):
    """Half the spacing of e4m3fn values around |x| <= 448 (2**-10 in the subnormal range)."""
    a = np.abs(x)
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (ex - 4)


def test_dequantized_q_nope_by_brute_force_and_error_bound():
    """ROCm/aiter PR #6199, Technical details: the query is quantized in-kernel
    to the fp8 range. Q' must equal the brute-force definition bit for bit and
    lie within half an e4m3fn step (times the row's 2**e) of q."""
    w = workloads.make("tiny", batch=2, s_q=2, h_q=8, seq_len=64, seed=5)
    bits = w.q_bits.copy()
    flat = bits.reshape(-1, bits.shape[-1])
    # special rows: all zero; amax 1e-37 (2**-e beyond float32's range); bf16
    # subnormals; an amax of exactly 448 * 2**3; a row of one large value
    tiny = np.float32(1e-37)
    flat[0, :512] = 0
    flat[1, :512] = (torch.from_numpy(np.linspace(-1, 1, 512, dtype=np.float32) * tiny)
                     .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    flat[2, :512] = np.arange(512, dtype=np.uint16) % 0x7F + 1          # positive bf16 subnormals
    flat[3, :512] = (torch.full((512,), 3.0).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    flat[3, 7] = torch.tensor([448.0 * 8]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]
    flat[4, :512] = 0
    flat[4, 100] = torch.tensor([-1.5e5]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]
    qp = attn.dequantized_q_nope(bits)
    q = fp8.bf16_bits_to_f64(bits)[..., :512]
    qp_f, q_f = qp.reshape(-1, 512), q.reshape(-1, 512)
    _, exps = attn.quantize_q_rows(q)
    for r in range(q_f.shape[0]):
        ref, e = _brute_force_q_prime(q_f[r])
        np.testing.assert_array_equal(qp_f[r], ref, err_msg=f"row {r}")
        assert exps.reshape(-1)[r] == e
        bound = _e4m3fn_half_step(q_f[r] * 2.0 ** -e) * 2.0 ** e
        assert np.all(np.abs(qp_f[r] - q_f[r]) <= bound), f"row {r}"
    assert np.all(qp_f[0] == 0)
    assert np.all(np.isfinite(qp_f)) and np.abs(qp_f[1]).max() > 0
    assert exps.reshape(-1)[3] == 3 and qp_f[3, 7] == 448.0 * 8
