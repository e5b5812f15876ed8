"""Pins of the quantize-on-write oracle (oracle/cache.py) against facts fixed
by the format and the scale rule (InfiniCore PR #1568, Summary, FP8 KV cache
bullet: per-tensor scale amax / 448), not against its own formulas."""

import numpy as np
import pytest
import torch

from oracle import cache, fp8


def _inputs(n, d_rope=64, pages=8, seed=0, scale_up=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, 512)) * scale_up).astype(np.float32)
    ckv = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rope = None
    if d_rope:
        r = rng.standard_normal((n, d_rope)).astype(np.float32)
        rope = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = rng.permutation(pages * 64)[:n].astype(np.int32)
    kv = np.full((pages, 64, 1, 512 + 2 * d_rope), 0xFF, dtype=np.uint8)
    return ckv, rope, slots, kv


def test_amax_element_encodes_to_448():
    ckv, rope, slots, kv = _inputs(40, seed=1)
    new, s = cache.quantize_kv(ckv, rope, slots, kv)
    vals = fp8.bf16_bits_to_f64(ckv)
    t, d = np.unravel_index(np.argmax(np.abs(vals)), vals.shape)
    code = new.reshape(-1, new.shape[-1])[slots[t], d]
    assert code == (0xFE if vals[t, d] < 0 else 0x7E)
    # and the scale is the f32 quotient amax / 448
    assert s == np.float32(np.float32(np.abs(vals).max()) / np.float32(448.0))


def test_codes_are_nearest_by_brute_force():
    ckv, rope, slots, kv = _inputs(6, seed=2)
    new, s = cache.quantize_kv(ckv, rope, slots, kv)
    rows = new.reshape(-1, new.shape[-1])
    finite = np.array([c for c in range(256) if not np.isnan(fp8.E4M3FN_TABLE[c])])
    vals = fp8.E4M3FN_TABLE[finite]
    x = fp8.bf16_bits_to_f64(ckv).astype(np.float32)
    for t in range(ckv.shape[0]):
        for d in range(0, 512, 7):
            q = float(np.float32(x[t, d] / s))
            q = min(max(q, -448.0), 448.0)
            dist = np.abs(vals - q)
            best = finite[dist == dist.min()]
            if len(best) > 1:   # tie: the even mantissa; for zero the sign of q
                best = [c for c in best if (c & 1) == 0 and ((c >> 7) == (q < 0) or fp8.E4M3FN_TABLE[c] != 0)]
            assert rows[slots[t], d] in best, (t, d, q)


def test_round_trip_within_half_step():
    ckv, rope, slots, kv = _inputs(30, seed=3)
    new, s = cache.quantize_kv(ckv, rope, slots, kv)
    rows = new.reshape(-1, new.shape[-1])
    x = fp8.bf16_bits_to_f64(ckv)
    back = fp8.decode_e4m3fn(rows[slots, :512]) * float(s)
    # e4m3fn: 3 mantissa bits (half step 2^-4 relative) for normals, absolute
    # half step 2^-10 below 2^-6 (subnormals), in units of the scale
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6)
    assert np.all(np.abs(back - x) <= bound)


def test_rope_and_untouched_rows_are_copied():
    ckv, rope, slots, kv = _inputs(20, seed=4)
    new, _ = cache.quantize_kv(ckv, rope, slots, kv)
    rows = new.reshape(-1, new.shape[-1])
    assert np.array_equal(rows[slots, 512:].view("<u2"), rope)
    untouched = np.setdiff1d(np.arange(rows.shape[0]), slots)
    assert np.all(rows[untouched] == 0xFF)


def test_skipped_tokens_do_not_count():
    ckv, rope, slots, kv = _inputs(10, seed=5)
    big = torch.full((1, 512), 1000.0).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ckv2 = np.concatenate([ckv, big])
    rope2 = np.concatenate([rope, rope[:1]])
    for bad in (-1, kv.shape[0] * 64, 10 ** 6):
        slots2 = np.concatenate([slots, [bad]]).astype(np.int32)
        new2, s2 = cache.quantize_kv(ckv2, rope2, slots2, kv)
        new1, s1 = cache.quantize_kv(ckv, rope, slots, kv)
        assert s1 == s2 and np.array_equal(new1, new2)


def test_slot_permutation_moves_rows_only():
    ckv, rope, slots, kv = _inputs(16, seed=6)
    new, s = cache.quantize_kv(ckv, rope, slots, kv)
    perm = np.random.default_rng(7).permutation(kv.shape[0] * 64)
    slots_p = perm[slots].astype(np.int32)
    new_p, s_p = cache.quantize_kv(ckv, rope, slots_p, kv)
    assert s == s_p
    r, rp = new.reshape(-1, new.shape[-1]), new_p.reshape(-1, new.shape[-1])
    assert np.array_equal(r[slots], rp[slots_p])


def test_given_scale_and_zero_amax():
    ckv, rope, slots, kv = _inputs(8, d_rope=0, seed=8)
    new, s = cache.quantize_kv(ckv, None, slots, kv, scale=np.float32(0.01))
    assert s == np.float32(0.01)
    assert np.array_equal(new.reshape(-1, 512)[slots], cache.encode_rows(ckv, np.float32(0.01)))
    zeros = np.zeros_like(ckv)
    _, s0 = cache.quantize_kv(zeros, None, slots, kv)
    assert s0 == np.float32(1.0)


@pytest.mark.parametrize("scale_up", [1.0, 1e-3, 50.0])
def test_codes_match_torch_float8_cast(scale_up):
    """Outside check: torch's float8_e4m3fn cast of the same f32 quotients."""
    ckv, rope, slots, kv = _inputs(12, seed=9, scale_up=scale_up)
    s = cache.kv_scale(ckv, slots, kv.shape[0] * 64)
    x = fp8.bf16_bits_to_f64(ckv).astype(np.float32)
    q = np.clip((x / s).astype(np.float32), -448.0, 448.0)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(cache.encode_rows(ckv, s), ref)



def test_per_token_quantize():
    """Each written token gets amax / 448 of its own row; its max element is
    +-448; other rows (cache and scales) are untouched."""
    ckv, rope, slots, kv = _inputs(24, seed=12)
    rng = np.random.default_rng(13)
    x = fp8.bf16_bits_to_f64(ckv) * rng.uniform(0.01, 10.0, (24, 1))
    ckv = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    scales0 = np.full((kv.shape[0], 64), -1.0, dtype=np.float32)
    new, sc = cache.quantize_kv_per_token(ckv, rope, slots, kv, scales0)
    rows = new.reshape(-1, new.shape[-1])
    vals = fp8.bf16_bits_to_f64(ckv)
    for t in range(24):
        st = sc.reshape(-1)[slots[t]]
        assert st == np.float32(np.float32(np.abs(vals[t]).max()) / np.float32(448.0))
        d = int(np.argmax(np.abs(vals[t])))
        assert rows[slots[t], d] == (0xFE if vals[t, d] < 0 else 0x7E)
        assert np.array_equal(rows[slots[t], :512], cache.encode_rows(ckv[t:t + 1], st)[0])
    untouched = np.setdiff1d(np.arange(rows.shape[0]), slots)
    assert np.all(sc.reshape(-1)[untouched] == -1.0) and np.all(rows[untouched] == 0xFF)
