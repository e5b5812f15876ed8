"""Seeded synthetic inputs for FP8-KV paged MLA decode.

This module only draws inputs: it holds none of the attention arithmetic and
imports neither the oracle nor the HIP library, so both sides can take their
inputs from here. Quantization of the synthetic latent to e4m3fn and of the
queries to bf16 uses torch's CPU casts (round to nearest even), a library
primitive independent of both sides.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, draws in
this order):

  dense  1. seq_lens (only when drawn, e.g. Uniform{2048..6144})
         2. Q ~ N(0,1) float32 [b, s_q, h_q, d_nope+d_rope] -> bf16
         3. latent ~ N(0,1) float32 [sum(seq_lens), d_nope]
         4. rope ~ N(0,1) float32 [sum(seq_lens), d_rope] -> bf16
         5. a permutation of the page pool, handing 64-token pages to
            (sequence, logical page) in order
  sparse 1. indices: per (b, i) topk distinct positions in [0, seq_len)
         2. latent ~ N(0,1) for the referenced rows only (sorted by position)
         3. noise ~ N(0,1) [b, s_q, h_q, d_nope] for the queries
         4. the page permutation
     The query of token (b, i) is gamma * xi_d + 0.05 * noise, xi_d being the
     latent row of the first index, gamma = 9 / (softmax_scale * |xi_d|^2):
     the first key scores about 9 above the rest, whose logits are roughly
     N(0, 0.4^2), so the tail carries about a fifth of the softmax mass.

The per-tensor scale is amax/448 over the valid latent (float32), and
k_scale = v_scale = that scale. Every byte of the pool that no valid token
owns (unused pages, the slack of each last page, unreferenced rows of the
sparse context) is 0xFF, a NaN in both e4m3fn and bf16, so a stray read
poisons the output. Unused block_table entries point at a poisoned page.
With ``encoding="e4m3fnuz"`` (gfx942's code, largest value 240) the latent
is cast to torch's float8_e4m3fnuz at scale amax/240, and the code columns
of unowned rows are 0x80, that encoding's NaN.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

PAGE_BLOCK = 64
POISON = 0xFF

#: The five workload configurations plus the benchmark shape ("metric").
SPECS = {
    # b=1, s_q=1, h_q=16, cache 256, num_splits=1
    "tiny": dict(batch=1, s_q=1, h_q=16, d_rope=64, seq_len=256, causal=True,
                 num_splits=1, dots=("bf16", "fp8")),
    # b=32, s_q=2 causal, h_q=64, cache 8196, shuffled pages, auto splits
    "mtp": dict(batch=32, s_q=2, h_q=64, d_rope=64, seq_len=8196, causal=True,
                num_splits=0, dots=("bf16", "fp8")),
    # b=64, s_q=2 causal, h_q=64, seq_lens ~ U{2048..6144}, fp8 dots
    "varlen": dict(batch=64, s_q=2, h_q=64, d_rope=64, seq_len=(2048, 6144),
                   causal=True, num_splits=0, dots=("fp8",)),
    # b=128, s_q=2, h_q=64, cache 8196, bf16 vs fp8 dots on the same inputs
    "large": dict(batch=128, s_q=2, h_q=64, d_rope=64, seq_len=8196, causal=True,
                  num_splits=0, dots=("bf16", "fp8")),
    # b=16, s_q=2, h_q=16, rope-free 512, context 131072, top-2048, peaky
    "sparse": dict(batch=16, s_q=2, h_q=16, d_rope=0, seq_len=131072, causal=False,
                   topk=2048, peaky=True, num_splits=0, dots=("bf16", "fp8")),
    # the benchmark shape: b=64, s_q=2, sk=8196, h_q=64 (built like "mtp")
    "metric": dict(batch=64, s_q=2, h_q=64, d_rope=64, seq_len=8196, causal=True,
                   num_splits=0, dots=("fp8", "bf16")),
    # 16-token sparse decode (the aiter PR's second workload, same model shard
    # as "sparse"): b=2 so that the token count (32) matches "sparse"
    "sparse16": dict(batch=2, s_q=16, h_q=16, d_rope=0, seq_len=131072, causal=False,
                     topk=2048, peaky=True, num_splits=0, dots=("bf16", "fp8")),
    # chunked prefill over the fp8 cache: the last 256 tokens of 4096-token
    # sequences attend causally to the whole cache (16 heads)
    "prefill": dict(batch=2, s_q=256, h_q=16, d_rope=64, seq_len=4096, causal=True,
                    num_splits=0, dots=("bf16", "fp8")),
    # sparse prefill (the aiter PR's third workload, same model shard): 16K
    # query tokens of one sequence, each with its own top-2048 of the 16K keys
    "sparse_prefill": dict(batch=1, s_q=16384, h_q=16, d_rope=0, seq_len=16384, causal=False,
                           topk=2048, peaky=True, num_splits=0, dots=("bf16", "fp8")),
    # the aiter PR's batch series (ROCm/aiter PR #6199, the bench commit: decode
    # at 1, 8 and 64 sequences, 16 heads, context 8192, top-k 2048): one query
    # token per sequence (a decode step), the same rope-free shard, random
    # (not peaky) queries
    "sparse_b1": dict(batch=1, s_q=1, h_q=16, d_rope=0, seq_len=8192, causal=False,
                      topk=2048, peaky=False, num_splits=0, dots=("bf16", "fp8")),
    "sparse_b8": dict(batch=8, s_q=1, h_q=16, d_rope=0, seq_len=8192, causal=False,
                      topk=2048, peaky=False, num_splits=0, dots=("bf16", "fp8")),
    "sparse_b64": dict(batch=64, s_q=1, h_q=16, d_rope=0, seq_len=8192, causal=False,
                       topk=2048, peaky=False, num_splits=0, dots=("bf16", "fp8")),
}

SEEDS = {"tiny": 1, "mtp": 2, "varlen": 3, "large": 4, "sparse": 5, "metric": 6, "sparse16": 7, "prefill": 8,
         "sparse_prefill": 9, "sparse_b1": 10, "sparse_b8": 11, "sparse_b64": 12}


@dataclass
class Workload:
    name: str
    batch: int
    s_q: int
    h_q: int
    d_nope: int
    d_rope: int
    causal: bool
    topk: int
    q_bits: np.ndarray            # uint16 bf16 [b, s_q, h_q, d_nope + d_rope]
    kv_cache: np.ndarray          # uint8 [num_pages, 64, row_bytes]
    block_table: np.ndarray       # int32 [b, max_pages]
    seq_lens: np.ndarray          # int32 [b]
    k_scale: float                # exact float32 value
    v_scale: float
    indices: Optional[np.ndarray] = None   # int32 [b, s_q, topk] (sparse only)
    num_splits: int = 0
    dots: Tuple[str, ...] = ("fp8",)
    page_block: int = PAGE_BLOCK
    softmax_scale: Optional[float] = None
    encoding: str = "e4m3fn"      # the cache's one-byte code: e4m3fn or gfx942's e4m3fnuz
    meta: dict = field(default_factory=dict)

    @property
    def row_bytes(self) -> int:
        return self.d_nope + 2 * self.d_rope

    @property
    def num_pages(self) -> int:
        return self.kv_cache.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


#: one-byte cache encodings: torch dtype of the cast, largest magnitude, and
#: the byte that poisons the code columns (a NaN of the encoding)
ENCODINGS = {"e4m3fn": (torch.float8_e4m3fn, 448.0, 0xFF),
             "e4m3fnuz": (torch.float8_e4m3fnuz, 240.0, 0x80)}


def _code_bytes(x: np.ndarray, encoding: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(ENCODINGS[encoding][0])
    return t.view(torch.uint8).numpy()


def _per_tensor_scale(latent: np.ndarray, qmax: float = 448.0) -> np.float32:
    amax = np.float32(np.abs(latent).max()) if latent.size else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(qmax))


def _encode_latent(latent: np.ndarray, spec) -> Tuple[np.ndarray, np.float32]:
    """Per-tensor scale (amax / the encoding's largest value) and the codes."""
    enc = spec.get("encoding", "e4m3fn")
    scale = _per_tensor_scale(latent, ENCODINGS[enc][1])
    return _code_bytes(latent / scale, enc), scale


def _poisoned_pool(pool: int, row_bytes: int, d_nope: int, spec) -> np.ndarray:
    cache = np.full((pool, PAGE_BLOCK, row_bytes), POISON, dtype=np.uint8)
    cache[:, :, :d_nope] = ENCODINGS[spec.get("encoding", "e4m3fn")][2]
    return cache


def make(name: str, seed: Optional[int] = None, **overrides) -> Workload:
    """Build a named workload; keyword overrides change its spec (e.g. batch=2)."""
    spec = dict(SPECS[name])
    spec.update(overrides)
    seed = SEEDS[name] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if spec.get("topk", 0):
        return _make_sparse(name, spec, rng)
    return _make_dense(name, spec, rng)


def _seq_lens(spec, rng) -> np.ndarray:
    sl = spec["seq_len"]
    b = spec["batch"]
    if isinstance(sl, tuple):
        return rng.integers(sl[0], sl[1] + 1, size=b).astype(np.int32)
    if isinstance(sl, (list, np.ndarray)):
        return np.asarray(sl, dtype=np.int32)
    return np.full(b, sl, dtype=np.int32)


def _page_pool(rng, pages_per_seq, extra_pages):
    """Shuffled page ids: block_table [b, max_pages] and the pool size."""
    total = int(pages_per_seq.sum())
    pool = total + extra_pages
    perm = rng.permutation(pool).astype(np.int32)
    max_pages = max(int(pages_per_seq.max()), 1)
    poison_page = perm[total] if extra_pages else 0
    bt = np.full((len(pages_per_seq), max_pages), poison_page, dtype=np.int32)
    k = 0
    for b, n in enumerate(pages_per_seq):
        bt[b, :n] = perm[k:k + n]
        k += n
    return bt, pool


def _make_dense(name, spec, rng) -> Workload:
    b, s_q, h_q = spec["batch"], spec["s_q"], spec["h_q"]
    d_nope, d_rope = spec.get("d_nope", 512), spec["d_rope"]
    seq_lens = _seq_lens(spec, rng)
    q = rng.standard_normal((b, s_q, h_q, d_nope + d_rope), dtype=np.float32)
    q_bits = _bf16_bits(q)
    ntok = int(seq_lens.sum())
    latent = rng.standard_normal((ntok, d_nope), dtype=np.float32)
    rope = rng.standard_normal((ntok, d_rope), dtype=np.float32)
    codes, scale = _encode_latent(latent, spec)
    del latent
    rope_bytes = _bf16_bits(rope).view(np.uint8).reshape(ntok, 2 * d_rope)
    pages_per_seq = -(-seq_lens.astype(np.int64) // PAGE_BLOCK)
    bt, pool = _page_pool(rng, pages_per_seq, spec.get("extra_pages", 2))
    row_bytes = d_nope + 2 * d_rope
    cache = _poisoned_pool(pool, row_bytes, d_nope, spec)
    t0 = 0
    for bi in range(b):
        n = int(seq_lens[bi])
        if n == 0:
            continue
        pos = np.arange(n)
        pages = bt[bi, pos // PAGE_BLOCK]
        slots = pos % PAGE_BLOCK
        cache[pages, slots, :d_nope] = codes[t0:t0 + n]
        if d_rope:
            cache[pages, slots, d_nope:] = rope_bytes[t0:t0 + n]
        t0 += n
    return Workload(name=name, batch=b, s_q=s_q, h_q=h_q, d_nope=d_nope, d_rope=d_rope,
                    causal=bool(spec["causal"]), topk=0, q_bits=q_bits, kv_cache=cache,
                    block_table=bt, seq_lens=seq_lens, k_scale=float(scale),
                    v_scale=float(scale), num_splits=spec.get("num_splits", 0),
                    dots=tuple(spec["dots"]), softmax_scale=spec.get("softmax_scale"),
                    encoding=spec.get("encoding", "e4m3fn"))


def _make_sparse(name, spec, rng) -> Workload:
    b, s_q, h_q = spec["batch"], spec["s_q"], spec["h_q"]
    d_nope, d_rope = spec.get("d_nope", 512), spec["d_rope"]
    topk = spec["topk"]
    seq_lens = _seq_lens(spec, rng)
    indices = np.empty((b, s_q, topk), dtype=np.int32)
    for bi in range(b):
        for i in range(s_q):
            n = int(seq_lens[bi])
            k = min(topk, n)
            indices[bi, i, :k] = rng.choice(n, size=k, replace=False)
            indices[bi, i, k:] = -1
    # latent rows for the referenced positions only
    ref = [np.unique(indices[bi][indices[bi] >= 0]) for bi in range(b)]
    nref = sum(len(r) for r in ref)
    latent = rng.standard_normal((nref, d_nope), dtype=np.float32)
    rope = rng.standard_normal((nref, d_rope), dtype=np.float32)
    sm = spec.get("softmax_scale") or 1.0 / np.sqrt(d_nope + d_rope)
    noise = rng.standard_normal((b, s_q, h_q, d_nope + d_rope), dtype=np.float32)
    q = np.empty((b, s_q, h_q, d_nope + d_rope), dtype=np.float32)
    offs = np.cumsum([0] + [len(r) for r in ref])
    for bi in range(b):
        for i in range(s_q):
            if spec.get("peaky", False) and indices[bi, i, 0] >= 0:
                row = offs[bi] + np.searchsorted(ref[bi], indices[bi, i, 0])
                xi = latent[row]
                gamma = np.float32(9.0 / (sm * float(np.dot(xi, xi))))
                q[bi, i, :, :d_nope] = gamma * xi[None, :] + np.float32(0.05) * noise[bi, i, :, :d_nope]
                q[bi, i, :, d_nope:] = noise[bi, i, :, d_nope:]
            else:
                q[bi, i] = noise[bi, i]
    q_bits = _bf16_bits(q)
    codes, scale = _encode_latent(latent, spec)
    rope_bytes = _bf16_bits(rope).view(np.uint8).reshape(nref, 2 * d_rope)
    pages_per_seq = -(-seq_lens.astype(np.int64) // PAGE_BLOCK)
    bt, pool = _page_pool(rng, pages_per_seq, spec.get("extra_pages", 2))
    row_bytes = d_nope + 2 * d_rope
    cache = _poisoned_pool(pool, row_bytes, d_nope, spec)
    for bi in range(b):
        pos = ref[bi].astype(np.int64)
        pages = bt[bi, pos // PAGE_BLOCK]
        slots = pos % PAGE_BLOCK
        cache[pages, slots, :d_nope] = codes[offs[bi]:offs[bi + 1]]
        if d_rope:
            cache[pages, slots, d_nope:] = rope_bytes[offs[bi]:offs[bi + 1]]
    return Workload(name=name, batch=b, s_q=s_q, h_q=h_q, d_nope=d_nope, d_rope=d_rope,
                    causal=False, topk=topk, q_bits=q_bits, kv_cache=cache,
                    block_table=bt, seq_lens=seq_lens, k_scale=float(scale),
                    v_scale=float(scale), indices=indices,
                    num_splits=spec.get("num_splits", 0), dots=tuple(spec["dots"]),
                    softmax_scale=spec.get("softmax_scale"),
                    encoding=spec.get("encoding", "e4m3fn"))


def flops(w: Workload) -> float:
    """Useful FLOPs of one call: 2 * rows * visible keys * (d + dv) summed over rows."""
    d, dv = w.d_nope + w.d_rope, w.d_nope
    keys = 0
    for b in range(w.batch):
        sk = int(w.seq_lens[b])
        for i in range(w.s_q):
            if w.indices is not None:
                idx = w.indices[b, i]
                n = int(((idx >= 0) & (idx < sk)).sum())
            else:
                n = max(sk - (w.s_q - 1 - i), 0) if w.causal else sk
            keys += n
    return 2.0 * w.h_q * keys * (d + dv)


def algorithmic_bytes(w: Workload) -> dict:
    """Bytes one call must move at least once: KV rows needed, Q, out, lse, tables."""
    if w.indices is not None:
        kv_rows = 0
        for b in range(w.batch):
            sk = int(w.seq_lens[b])
            for i in range(w.s_q):
                idx = w.indices[b, i]
                kv_rows += int(((idx >= 0) & (idx < sk)).sum())
        tables = w.indices.nbytes + w.block_table.nbytes + w.seq_lens.nbytes
    else:
        kv_rows = int(w.seq_lens.sum())
        pages = int((-(-w.seq_lens.astype(np.int64) // w.page_block)).sum())
        tables = 4 * pages + w.seq_lens.nbytes
    kv = kv_rows * w.row_bytes
    q = w.q_bits.nbytes
    out = w.batch * w.s_q * w.h_q * w.d_nope * 2
    lse = w.batch * w.s_q * w.h_q * 4
    return dict(kv=kv, q=q, out=out, lse=lse, tables=tables, total=kv + q + out + lse + tables)
