"""Float64 MLA decode over a paged FP8 e4m3fn KV cache (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages fix it:

* One shared latent KV head per token (h_kv = 1): d = 576 = 512 e4m3fn "nope"
  dims plus 64 rope dims kept in bf16; V is the 512-wide latent, dv = 512
  (FlashMLA PR #82 "update fp8 support": description, the nine 64-wide Q@K
  tiles with the rope tile in BF16, and the test report's
  h_kv=1, d=576, dv=512, causal=True parameters).
* Per-tensor k/v scales on the fp8 part; the cache is quantized with
  scale = amax/448 (InfiniCore PR #1568, Summary, FP8 KV cache bullet). The
  per-token variant the same page names (scales [num_blocks, h_kv,
  block_size]) takes one k and one v scale per cache row (scale_at).
* "f32 attention over the same fp8 cache" is the accuracy reference
  (ROCm/aiter PR #6199, Results, Accuracy paragraph): here in float64.
* Split-KV flash decoding: each split yields a partial (max, sum of exps,
  weighted sum) and a second pass merges them; empty shards publish the
  neutral element and the merge guards it (InfiniCore PR #1568, split-kv
  commit and the len-0 fix commit). Here the partial is carried as
  (o_s = normalised output, lse_s), which is the same information.
* Rows with no visible key give zeros (InfiniCore PR #1568, len-0 fix commit;
  FlashInfer PR #1769 review: a fully masked row must not average V); their
  lse is -inf.
* The fp8-dot path quantizes Q inside the kernel to the fp8 range
  (ROCm/aiter PR #6199, Technical details). The granularity and rounding are
  not given; the reading taken here is one power-of-two scale per query row
  over the 512 nope dims, the smallest 2**e with amax <= 448 * 2**e
  (2**0 when the row is all zero), then round-to-nearest-even e4m3fn.

Readings where the pages are silent (each is listed in the design doc):
  softmax scale 1/sqrt(d_nope + d_rope); causal rows aligned bottom-right
  (query token i of s_q sees keys 0 .. sk - s_q + i); lse in natural log;
  k_scale does not touch the bf16 rope dims; V = the dequantized nope dims
  times v_scale; sparse indices are logical positions inside the sequence
  (mapped through block_table), entries < 0 or >= seq_len are skipped, and
  sparse rows take no causal mask.

Pins (tests/test_oracle_attn.py): closed forms (equal logits give the mean of
V and lse = ln L; a dominant key gives its own V row; the one-key-plus-tail
fixture gives tail share 2047 e^-9 / (1 + 2047 e^-9)), brute-force scalar
loops on tiny inputs, split invariance over 1..8 splits including empty ones,
block_table permutation invariance and v_scale linearity.
"""

import math

import numpy as np

from .fp8 import E4M3FN_MAX, bf16_bits_to_f64, decode_e4m3fn, decode_kv_codes, encode_e4m3fn


def default_softmax_scale(d_nope: int, d_rope: int) -> float:
    return 1.0 / math.sqrt(d_nope + d_rope)


def _positions_to_rows(kv_cache, block_table_row, pos, page_block):
    pages = block_table_row[pos // page_block]
    slots = pos % page_block
    return kv_cache[pages, slots]  # [n, row_bytes] uint8


def scale_at(scale, block_table_row, pos, page_block=64):
    """The scale of each key position: a per-tensor scale (a scalar) as is, or
    per-token scales (an array [pages, page_block], one per cache row) looked
    up at the positions' rows (InfiniCore PR #1568, Summary: the per-token
    scale layout [num_blocks, h_kv, block_size])."""
    s = np.asarray(scale, dtype=np.float64)
    if s.size == 1:
        return float(s.reshape(-1)[0])
    pos = np.asarray(pos, dtype=np.int64)
    pages = np.asarray(block_table_row)[pos // page_block]
    return s.reshape(-1, page_block)[pages, pos % page_block]


def dequant_keys_values(rows, k_scale, v_scale, d_nope, d_rope, encoding="e4m3fn"):
    """Cache rows (uint8 [n, row_bytes]) -> K float64 [n, d_nope+d_rope], V [n, d_nope].

    Row layout: d_nope one-byte codes (e4m3fn, or gfx942's e4m3fnuz), then
    d_rope little-endian bf16 values. The scales are scalars or one value per
    row ([n], see scale_at).
    """
    nope = decode_kv_codes(rows[:, :d_nope], encoding)
    ks = np.asarray(k_scale, dtype=np.float64)
    vs = np.asarray(v_scale, dtype=np.float64)
    k = nope * (ks[:, None] if ks.ndim else float(ks))
    v = nope * (vs[:, None] if vs.ndim else float(vs))
    if d_rope:
        rb = np.ascontiguousarray(rows[:, d_nope:d_nope + 2 * d_rope])
        rope = bf16_bits_to_f64(rb.view("<u2"))
        k = np.concatenate([k, rope], axis=1)
    return k, v


def visible_positions(b, i, seq_lens, s_q, causal, indices=None):
    """Logical key positions query token i of sequence b attends to."""
    sk = int(seq_lens[b])
    if indices is not None:
        idx = np.asarray(indices[b, i]).astype(np.int64)
        return idx[(idx >= 0) & (idx < sk)]
    n = sk - (s_q - 1 - i) if causal else sk
    return np.arange(max(n, 0), dtype=np.int64)


def _attend(qrows, k, v, scale):
    """Softmax attention of query rows [h, d] over keys k [n, d], values v [n, dv]."""
    h = qrows.shape[0]
    if k.shape[0] == 0:
        return np.zeros((h, v.shape[1])), np.full(h, -np.inf)
    z = scale * (qrows @ k.T)                      # [h, n]
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    l = w.sum(axis=1, keepdims=True)
    out = (w @ v) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def query_f64(q_bits, q_nope_override=None, d_nope=512):
    """bf16 query bits [b, s_q, h_q, d] -> float64, optionally with the nope dims replaced."""
    q = bf16_bits_to_f64(q_bits)
    if q_nope_override is not None:
        q = q.copy()
        q[..., :d_nope] = q_nope_override
    return q


def mla_decode(q_bits, kv_cache, block_table, seq_lens, k_scale, v_scale, *,
               d_nope=512, d_rope=64, causal=True, softmax_scale=None,
               indices=None, q_nope_override=None, page_block=64, batches=None, encoding="e4m3fn"):
    """Attention of every (b, i, h) query row over its visible keys.

    Arguments are host arrays in the library's layouts: q_bits uint16 bf16
    [b, s_q, h_q, d_nope+d_rope]; kv_cache uint8 [pages, page_block, row_bytes]
    (the h_kv = 1 axis squeezed); block_table int32 [b, max_pages]; seq_lens
    int32 [b]; indices int32 [b, s_q, topk] for the sparse variant.
    ``q_nope_override`` (float64 [b, s_q, h_q, d_nope]) replaces the nope part
    of the query; pass the dequantized Q' to get the fp8-dot path's logits.
    ``batches`` restricts the work to those sequence indices (others stay 0).
    ``encoding`` names the cache's one-byte code ("e4m3fn" or "e4m3fnuz").

    Returns out float64 [b, s_q, h_q, d_nope] and lse float64 [b, s_q, h_q].
    """
    q = query_f64(q_bits, q_nope_override, d_nope)
    nb, s_q, h_q, _ = q.shape
    scale = default_softmax_scale(d_nope, d_rope) if not softmax_scale else softmax_scale
    out = np.zeros((nb, s_q, h_q, d_nope))
    lse = np.full((nb, s_q, h_q), -np.inf)
    for b in (range(nb) if batches is None else batches):
        if indices is None:
            # every token of the sequence reads a prefix of the same key list
            full = visible_positions(b, s_q - 1, seq_lens, s_q, False)
            rows = _positions_to_rows(kv_cache, block_table[b], full, page_block)
            k_all, v_all = dequant_keys_values(rows, scale_at(k_scale, block_table[b], full, page_block),
                                               scale_at(v_scale, block_table[b], full, page_block),
                                               d_nope, d_rope, encoding)
        for i in range(s_q):
            pos = visible_positions(b, i, seq_lens, s_q, causal, indices)
            if indices is None:
                k, v = k_all[:len(pos)], v_all[:len(pos)]
            else:
                rows = _positions_to_rows(kv_cache, block_table[b], pos, page_block)
                k, v = dequant_keys_values(rows, scale_at(k_scale, block_table[b], pos, page_block),
                                           scale_at(v_scale, block_table[b], pos, page_block), d_nope, d_rope,
                                           encoding)
            out[b, i], lse[b, i] = _attend(q[b, i], k, v, scale)
    return out, lse


def split_ranges(n_units, num_splits):
    """Contiguous, balanced unit ranges [lo, hi) for each split (some may be empty)."""
    return [(s * n_units // num_splits, (s + 1) * n_units // num_splits)
            for s in range(num_splits)]


def split_partials(q_bits, kv_cache, block_table, seq_lens, k_scale, v_scale,
                   num_splits, *, d_nope=512, d_rope=64, causal=True,
                   softmax_scale=None, indices=None, q_nope_override=None,
                   page_block=64, encoding="e4m3fn"):
    """Split-KV partials: per split s, (o_s, lse_s) over that split's keys.

    Dense: the sequence's pages are cut into ``num_splits`` contiguous,
    page-aligned ranges. Sparse: the index list is cut the same way in units
    of 64 entries. A split with no visible key for a row gives (0, -inf).
    ``encoding`` names the cache's one-byte code, as for mla_decode.
    Returns o [S, b, s_q, h_q, d_nope], lse [S, b, s_q, h_q].
    """
    q = query_f64(q_bits, q_nope_override, d_nope)
    nb, s_q, h_q, _ = q.shape
    scale = default_softmax_scale(d_nope, d_rope) if not softmax_scale else softmax_scale
    o = np.zeros((num_splits, nb, s_q, h_q, d_nope))
    lse = np.full((num_splits, nb, s_q, h_q), -np.inf)
    for b in range(nb):
        sk = int(seq_lens[b])
        for i in range(s_q):
            if indices is None:
                vis = visible_positions(b, i, seq_lens, s_q, causal)
                n_units = -(-sk // page_block)
                for s, (lo, hi) in enumerate(split_ranges(n_units, num_splits)):
                    pos = vis[(vis >= lo * page_block) & (vis < hi * page_block)]
                    rows = _positions_to_rows(kv_cache, block_table[b], pos, page_block)
                    k, v = dequant_keys_values(rows, scale_at(k_scale, block_table[b], pos, page_block),
                                               scale_at(v_scale, block_table[b], pos, page_block),
                                               d_nope, d_rope, encoding)
                    o[s, b, i], lse[s, b, i] = _attend(q[b, i], k, v, scale)
            else:
                entries = np.asarray(indices[b, i]).astype(np.int64)
                n_units = -(-len(entries) // 64)
                for s, (lo, hi) in enumerate(split_ranges(n_units, num_splits)):
                    part = entries[lo * 64:hi * 64]
                    pos = part[(part >= 0) & (part < sk)]
                    rows = _positions_to_rows(kv_cache, block_table[b], pos, page_block)
                    k, v = dequant_keys_values(rows, scale_at(k_scale, block_table[b], pos, page_block),
                                               scale_at(v_scale, block_table[b], pos, page_block),
                                               d_nope, d_rope, encoding)
                    o[s, b, i], lse[s, b, i] = _attend(q[b, i], k, v, scale)
    return o, lse


def combine(o_parts, lse_parts):
    """Log-sum-exp merge of split partials along axis 0.

    lse = log sum_s exp(lse_s) (max-subtracted; all -inf gives -inf);
    out = sum_s exp(lse_s - lse) * o_s (all -inf gives 0).
    """
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, wsum, 1.0)), -np.inf)
    wn = np.where(finite[None], w / np.where(finite, wsum, 1.0)[None], 0.0)
    out = (wn[..., None] * o_parts).sum(axis=0)
    return out, lse


def q_row_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2**e (0 for amax == 0)."""
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 10          # 448 * 2**e < 2**(e+9): start low
    while amax > E4M3FN_MAX * 2.0 ** e:
        e += 1
    return e


def quantize_q_rows(q_nope):
    """Per-row power-of-two e4m3fn quantization of the query's nope dims.

    q_nope float64 [..., d_nope] (exact bf16 values). Returns (codes uint8
    [..., d_nope], exps int32 [...]) with q_nope ~= decode(codes) * 2**exps.
    """
    q = np.asarray(q_nope, dtype=np.float64)
    flat = q.reshape(-1, q.shape[-1])
    exps = np.array([q_row_exponent(float(np.abs(r).max())) for r in flat], dtype=np.int32)
    codes = encode_e4m3fn(flat * np.ldexp(1.0, -exps.astype(np.int64))[:, None])
    return codes.reshape(q.shape), exps.reshape(q.shape[:-1])


def dequantized_q_nope(q_bits, d_nope=512):
    """Q' (the fp8-dot path's query, dequantized) as float64 [..., d_nope].

    Each row's nope part is quantized as quantize_q_rows does (the query
    quantized in-kernel to the fp8 range, ROCm/aiter PR #6199, Technical
    details) and mapped back: Q' = decode(code) * 2**e, so that |Q' - q| is at
    most half an e4m3fn step at q's magnitude times 2**e.
    """
    codes, exps = quantize_q_rows(bf16_bits_to_f64(q_bits)[..., :d_nope])
    return decode_e4m3fn(codes) * np.ldexp(1.0, exps.astype(np.int64))[..., None]
