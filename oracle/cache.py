"""Quantize-on-write of the paged FP8 latent cache (reference form).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The step that fills the cache the decode reads (InfiniCore PR #1568,
Summary, FP8 KV cache bullet: per-tensor scale amax / 448, 448 being the
largest finite e4m3fn value). Readings where the page is silent:
  * the scale is per call ("per tensor"): the amax runs over the 512 nope
    values of the tokens actually written (a negative or out-of-range slot
    is not written and does not count); rope values stay bf16 and do not
    count; an amax of 0 gives scale 1;
  * arithmetic is float32, as the kernel's: scale = f32(amax) / f32(448),
    each value x / scale as one correctly rounded f32 division, clamped to
    [-448, 448], then rounded to the nearest e4m3fn code, ties to even
    (fp8.encode_e4m3fn, which is exact on an f32 input);
  * a token's cache row is slot = page * 64 + position in the page (the
    caller's slot mapping); the row keeps the decode's byte layout: 512 codes,
    then the rope values' little-endian bf16 bytes.

quantize_kv_per_token is the per-token variant (InfiniCore PR #1568,
Summary: scales laid out [num_blocks, h_kv, block_size]): one scale per
written row, amax of that row / 448.

Pinned by tests/test_oracle_cache.py: the amax element encodes to +-448
exactly; every other code is the nearest code of its f32 quotient (brute
force over all 256 codes); decode(code) * scale reproduces x to half a code
step; rope bytes and untouched rows are copied unchanged; skipped tokens do
not enter the scale; a permutation of the slots moves rows and nothing else.
"""

import numpy as np

from . import fp8

E4M3FN_MAX_F32 = np.float32(448.0)


def kv_scale(ckv_bits, slot_mapping, num_rows):
    """f32 per-tensor scale over the written tokens (amax / 448; 1 if amax = 0)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    ok = (slots >= 0) & (slots < num_rows)
    vals = fp8.bf16_bits_to_f64(np.asarray(ckv_bits)[ok])
    amax = np.float32(np.abs(vals).max()) if vals.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / E4M3FN_MAX_F32)


def encode_rows(ckv_bits, scale):
    """e4m3fn codes [n, 512] of the nope values under a given f32 scale."""
    x = fp8.bf16_bits_to_f64(np.asarray(ckv_bits)).astype(np.float32)
    q = (x / np.float32(scale)).astype(np.float32)
    q = np.clip(q, -E4M3FN_MAX_F32, E4M3FN_MAX_F32)
    return fp8.encode_e4m3fn(q.astype(np.float64))


def quantize_kv(ckv_bits, rope_bits, slot_mapping, kv_cache, scale=None):
    """Writes the tokens into a copy of kv_cache [pages, 64, 1, row] (uint8).

    ckv_bits: uint16 [n, 512]; rope_bits: uint16 [n, d_rope] or None;
    slot_mapping: int [n]; scale: None (compute amax / 448) or a given f32.
    Returns (new_cache, scale_used).
    """
    cache = np.array(kv_cache, dtype=np.uint8, copy=True)
    pages, blk = cache.shape[0], cache.shape[1]
    rows = cache.reshape(pages * blk, -1)
    n = np.asarray(slot_mapping).shape[0]
    if scale is None:
        scale = kv_scale(ckv_bits, slot_mapping, pages * blk)
    scale = np.float32(scale)
    if n == 0:
        return cache, scale
    codes = encode_rows(ckv_bits, scale)
    for t in range(n):
        s = int(slot_mapping[t])
        if s < 0 or s >= pages * blk:
            continue
        rows[s, :512] = codes[t]
        if rope_bits is not None and rope_bits.shape[1] > 0:
            rows[s, 512:] = np.asarray(rope_bits[t], dtype="<u2").view(np.uint8)
    return cache, scale


def quantize_kv_per_token(ckv_bits, rope_bits, slot_mapping, kv_cache, scales):
    """Per-token variant: every written token gets its own f32 scale, the
    amax of its 512 nope values / 448 (1 if that amax is 0), stored at its
    cache row in a copy of ``scales`` (f32, one per cache row; the k and v
    scales of a row are the same value). Returns (new_cache, new_scales)."""
    cache = np.array(kv_cache, dtype=np.uint8, copy=True)
    sc = np.array(scales, dtype=np.float32, copy=True).reshape(-1)
    pages, blk = cache.shape[0], cache.shape[1]
    rows = cache.reshape(pages * blk, -1)
    ckv_bits = np.asarray(ckv_bits)
    for t in range(np.asarray(slot_mapping).shape[0]):
        s = int(slot_mapping[t])
        if s < 0 or s >= pages * blk:
            continue
        amax = np.float32(np.abs(fp8.bf16_bits_to_f64(ckv_bits[t])).max())
        st = np.float32(amax / E4M3FN_MAX_F32) if amax > 0 else np.float32(1.0)
        rows[s, :512] = encode_rows(ckv_bits[t:t + 1], st)[0]
        if rope_bits is not None and rope_bits.shape[1] > 0:
            rows[s, 512:] = np.asarray(rope_bits[t], dtype="<u2").view(np.uint8)
        sc[s] = st
    return cache, sc.reshape(np.asarray(scales).shape)
