"""GPU parity of the quantize-on-write kernels (through the C ABI) with the
oracle (oracle/cache.py). Byte path: the cache bytes and the f32 scale must be
bit-exact."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
from oracle import cache

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _case(n, d_rope=64, pages=None, seed=0, scale_up=1.0, skip=0):
    rng = np.random.default_rng(seed)
    pages = pages or max(1, (n + skip + 63) // 64 + 2)
    ckv = _bf16_bits(rng.standard_normal((n, 512)) * scale_up)
    rope = _bf16_bits(rng.standard_normal((n, d_rope))) if d_rope else None
    slots = rng.permutation(pages * 64)[:n].astype(np.int32)
    if skip:
        bad = rng.choice(n, size=skip, replace=False)
        slots[bad[: skip // 2]] = -1
        slots[bad[skip // 2:]] = pages * 64 + 5
    kv = np.full((pages, 64, 1, 512 + 2 * d_rope), 0xFF, dtype=np.uint8)
    return ckv, rope, slots, kv


def _gpu(ckv, rope, slots, kv, scale=None):
    dev = "cuda:0"
    c = torch.from_numpy(ckv.view(np.int16)).view(torch.bfloat16).to(dev)
    r = None if rope is None else torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).to(dev)
    s = torch.from_numpy(slots).to(dev)
    k = torch.from_numpy(kv).to(dev)
    ks = torch.tensor([0.0 if scale is None else float(scale)], dtype=torch.float32, device=dev)
    vs = torch.tensor([-1.0], dtype=torch.float32, device=dev)
    mla.quantize_kv(c, r, s, k, ks, vs, compute_scale=scale is None)
    torch.cuda.synchronize()
    return k.cpu().numpy(), np.float32(ks.item()), np.float32(vs.item())


@pytest.mark.parametrize("n,d_rope,seed,scale_up,skip", [
    (1, 64, 1, 1.0, 0),
    (777, 64, 2, 1.0, 0),           # ragged: not a multiple of anything
    (4096, 64, 3, 3e-3, 0),         # small values: subnormal codes
    (3000, 0, 4, 20.0, 0),          # rope-free rows
    (2500, 64, 5, 1.0, 300),        # skipped and out-of-range slots
])
def test_quantize_matches_oracle(n, d_rope, seed, scale_up, skip):
    ckv, rope, slots, kv = _case(n, d_rope, seed=seed, scale_up=scale_up, skip=skip)
    ref, ref_s = cache.quantize_kv(ckv, rope, slots, kv)
    got, ks, vs = _gpu(ckv, rope, slots, kv)
    assert ks.view(np.uint32) == ref_s.view(np.uint32) and vs.view(np.uint32) == ref_s.view(np.uint32)
    assert np.array_equal(got, ref)


def test_quantize_given_scale():
    ckv, rope, slots, kv = _case(1000, 64, seed=6)
    ref, _ = cache.quantize_kv(ckv, rope, slots, kv, scale=np.float32(0.0071))
    got, ks, vs = _gpu(ckv, rope, slots, kv, scale=np.float32(0.0071))
    assert ks == np.float32(0.0071) and vs == np.float32(-1.0)   # scales not written
    assert np.array_equal(got, ref)


def test_quantize_no_tokens_sets_unit_scale():
    ckv, rope, slots, kv = _case(0, 64, pages=2, seed=7)
    got, ks, vs = _gpu(ckv, rope, slots, kv)
    assert ks == 1.0 and vs == 1.0 and np.array_equal(got, kv)


def test_quantize_full_cache_of_the_benchmark_shape():
    """64 sequences x 8196 tokens in shuffled pages (the decode benchmark's
    cache, written in one call): scale exact, and rows sampled across the
    cache bit-exact against the oracle's encoding of the same rows."""
    b, sk = 64, 8196
    ppseq = (sk + 63) // 64
    pages = b * ppseq
    rng = np.random.default_rng(11)
    n = b * sk
    ckv = _bf16_bits(rng.standard_normal((n, 512), dtype=np.float32))
    rope = _bf16_bits(rng.standard_normal((n, 64), dtype=np.float32))
    perm = rng.permutation(pages).astype(np.int64)
    pos = np.arange(sk)
    slots = np.concatenate([perm[s * ppseq + pos // 64] * 64 + pos % 64 for s in range(b)]).astype(np.int32)
    kv = np.full((pages, 64, 1, 640), 0xFF, dtype=np.uint8)
    got, ks, _ = _gpu(ckv, rope, slots, kv)
    ref_s = cache.kv_scale(ckv, slots, pages * 64)
    assert ks.view(np.uint32) == ref_s.view(np.uint32)
    pick = rng.choice(n, size=4096, replace=False)
    rows = got.reshape(-1, 640)
    assert np.array_equal(rows[slots[pick], :512], cache.encode_rows(ckv[pick], ref_s))
    assert np.array_equal(rows[slots[pick], 512:].view("<u2"), rope[pick])
    # the slack rows of every sequence's last page stay untouched
    used = np.zeros(pages * 64, dtype=bool)
    used[slots] = True
    assert np.all(rows[~used] == 0xFF)


def test_quantized_cache_decodes_like_the_oracle():
    """End to end: the cache written by the quantize kernel, decoded by the
    decode kernel, against the oracle decode of the oracle-written cache
    (the two caches are compared byte for byte first)."""
    from oracle import attn
    rng = np.random.default_rng(21)
    b, s_q, h_q, sk = 3, 2, 64, 700
    ppseq = (sk + 63) // 64
    pages = b * ppseq + 3
    perm = rng.permutation(pages)[: b * ppseq].reshape(b, ppseq).astype(np.int32)
    n = b * sk
    ckv = _bf16_bits(rng.standard_normal((n, 512)))
    rope = _bf16_bits(rng.standard_normal((n, 64)))
    pos = np.arange(sk)
    slots = np.concatenate([perm[s, pos // 64] * 64 + pos % 64 for s in range(b)]).astype(np.int32)
    kv0 = np.full((pages, 64, 1, 640), 0xFF, dtype=np.uint8)
    ref_cache, ref_s = cache.quantize_kv(ckv, rope, slots, kv0)
    got_cache, ks, vs = _gpu(ckv, rope, slots, kv0)
    assert ks.view(np.uint32) == ref_s.view(np.uint32) and np.array_equal(got_cache, ref_cache)
    q_bits = _bf16_bits(rng.standard_normal((b, s_q, h_q, 576)))
    seq_lens = np.full(b, sk, dtype=np.int32)
    ref_o, ref_l = attn.mla_decode(q_bits, ref_cache.reshape(pages, 64, 640), perm, seq_lens, float(ref_s),
                                   float(ref_s), causal=True)
    dev = "cuda:0"
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(got_cache).to(dev)
    bt = torch.from_numpy(perm).to(dev)
    sl = torch.from_numpy(seq_lens).to(dev)
    kst = torch.tensor([float(ks)], dtype=torch.float32, device=dev)
    vst = torch.tensor([float(vs)], dtype=torch.float32, device=dev)
    out, lse = mla.decode(q, kv, bt, sl, kst, vst, num_splits=0, dot="bf16", causal=True)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    rel = np.linalg.norm(o - ref_o) / np.linalg.norm(ref_o)
    assert rel <= 5e-3 and np.abs(lse.cpu().numpy() - ref_l).max() <= 1e-3


# Given scales for the every-value check: powers of two (every quotient exact,
# ties of the e4m3fn grid included), inexact ones, a scale under which most
# values saturate, and the ends of the range where the encoder changes from
# the reciprocal form to the division (2^-100 and 2^100 take the reciprocal,
# 1e-31 and 1e31 the division).
EVERY_VALUE_SCALES = [2.0 ** -7, 1.0, 0.0071, 1.0 / 3.0, 1.7e-3, 3.0, 1e-30, 1e30,
                      2.0 ** -100, 2.0 ** 100, 1e-31, 1e31, 0.013671875, 6.02e-5]


@pytest.mark.parametrize("scale", EVERY_VALUE_SCALES)
def test_quantize_every_bf16_value(scale):
    """Every finite and infinite bf16 bit pattern (128 tokens of 512 values;
    NaN patterns replaced by zero: the oracle gives them no code) encoded
    under a given scale, byte for byte as the oracle's correctly rounded f32
    division followed by saturation and round-to-nearest-even e4m3fn."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    nan = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
    bits[nan] = 0
    rng = np.random.default_rng(77)
    ckv = bits[rng.permutation(65536)].reshape(128, 512)
    rope = _bf16_bits(rng.standard_normal((128, 64)))
    pages = 3
    slots = rng.permutation(pages * 64)[:128].astype(np.int32)
    kv = np.full((pages, 64, 1, 640), 0xFF, dtype=np.uint8)
    sc = np.float32(scale)
    ref, _ = cache.quantize_kv(ckv, rope, slots, kv, scale=sc)
    got, ks, _ = _gpu(ckv, rope, slots, kv, scale=sc)
    assert ks.view(np.uint32) == sc.view(np.uint32)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"scale {scale}: {len(bad)} bytes differ, first at {bad[:4].tolist()}"


def test_quantize_per_token_every_bf16_value():
    """Per-token scales over every finite bf16 value: the non-NaN patterns
    sorted by magnitude and cut into rows of 512, each row then given half of
    another, smaller row's values (so quotients span many binades below the
    row's amax / scale = 448); rows whose amax makes the scale leave
    [2^-100, 2^100] take the division form, the others the reciprocal form.
    Cache bytes and per-row scales byte for byte as the oracle's."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    vals = bits[finite]
    mag = np.abs(torch.from_numpy(vals.view(np.int16)).view(torch.bfloat16).float().numpy())
    vals = vals[np.argsort(mag, kind="stable")]
    n = len(vals) // 512
    rows = vals[: n * 512].reshape(n, 512).copy()
    rng = np.random.default_rng(78)
    for r in range(1, n):
        j = int(rng.integers(0, r))
        take = rng.choice(512, size=256, replace=False)
        rows[r, take] = rows[j, rng.choice(512, size=256, replace=False)]
    rows = np.ascontiguousarray(rows[:, rng.permutation(512)])
    rope = _bf16_bits(rng.standard_normal((n, 64)))
    pages = (n + 63) // 64 + 1
    slots = rng.permutation(pages * 64)[:n].astype(np.int32)
    kv0 = np.full((pages, 64, 1, 640), 0xFF, dtype=np.uint8)
    sc0 = np.zeros((pages, 64), dtype=np.float32)
    ref_cache, ref_sc = cache.quantize_kv_per_token(rows, rope, slots, kv0, sc0)
    dev = "cuda:0"
    kv = torch.from_numpy(kv0).to(dev)
    ks = torch.from_numpy(sc0).to(dev)
    vs = torch.from_numpy(sc0).to(dev)
    mla.quantize_kv(torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to(dev),
                    torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).to(dev),
                    torch.from_numpy(slots).to(dev), kv, ks, vs, compute_scale="per_token")
    torch.cuda.synchronize()
    scales = ref_sc.reshape(-1)[slots]
    assert (scales < 2.0 ** -100).any() and ((scales >= 2.0 ** -100) & (scales <= 2.0 ** 100)).any()
    bad = np.argwhere(kv.cpu().numpy() != ref_cache)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:4].tolist()}"
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), ref_sc.view(np.uint32))
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), ref_sc.view(np.uint32))
