"""The seeded input generators: determinism, layout and the recipe's properties."""

import numpy as np
import torch

import workloads


def _valid_rows(w):
    rows = []
    for b in range(w.batch):
        pos = np.arange(int(w.seq_lens[b]))
        rows.append(w.kv_cache[w.block_table[b, pos // 64], pos % 64])
    return np.concatenate(rows)


def test_same_seed_same_bytes_and_different_seed_differs():
    a = workloads.make("tiny", batch=2, seq_len=[100, 30])
    b = workloads.make("tiny", batch=2, seq_len=[100, 30])
    c = workloads.make("tiny", batch=2, seq_len=[100, 30], seed=99)
    assert np.array_equal(a.kv_cache, b.kv_cache) and np.array_equal(a.q_bits, b.q_bits)
    assert not np.array_equal(a.q_bits, c.q_bits)


def test_dense_layout_poison_and_scale():
    w = workloads.make("mtp", batch=3, seq_len=[8196, 65, 1])
    assert w.kv_cache.shape[1:] == (64, 640) and w.q_bits.shape == (3, 2, 64, 576)
    pages = [-(-int(s) // 64) for s in w.seq_lens]
    used = np.concatenate([w.block_table[b, :n] for b, n in enumerate(pages)])
    assert len(np.unique(used)) == len(used) == sum(pages)
    # slack of a last page and every unused page are 0xFF
    assert np.all(w.kv_cache[w.block_table[0, 128], 4:] == 0xFF)
    assert np.all(w.kv_cache[w.block_table[2, 0], 1:] == 0xFF)
    unused = np.setdiff1d(np.arange(w.num_pages), used)
    assert len(unused) >= 1 and np.all(w.kv_cache[unused] == 0xFF)
    assert np.all(np.isin(w.block_table[1, 2:], unused))
    # scale = amax/448: the largest valid code is exactly 448 in magnitude
    codes = _valid_rows(w)[:, :512]
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    assert np.isfinite(vals).all() and np.abs(vals).max() == 448.0
    assert w.k_scale == w.v_scale and w.k_scale == float(np.float32(w.k_scale))
    rope = _valid_rows(w)[:, 512:].copy().view(np.uint16)
    assert np.isfinite(torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).float().numpy()).all()


def test_varlen_lengths_in_range():
    w = workloads.make("varlen", batch=64, seq_len=(2048, 6144))
    assert w.seq_lens.min() >= 2048 and w.seq_lens.max() <= 6144
    assert 3500 < w.seq_lens.mean() < 4700


def test_sparse_indices_unique_and_tail_mass_about_a_fifth():
    w = workloads.make("sparse", batch=2, seq_len=131072)
    assert w.indices.shape == (2, 2, 2048) and w.kv_cache.shape[2] == 512
    for b in range(2):
        for i in range(2):
            idx = w.indices[b, i]
            assert len(np.unique(idx)) == 2048 and idx.min() >= 0 and idx.max() < 131072
    # logits relative to the first (dominant) key, in float64 from torch decodes
    b, i = 1, 0
    idx = w.indices[b, i].astype(np.int64)
    rows = w.kv_cache[w.block_table[b, idx // 64], idx % 64]
    k = torch.from_numpy(rows.copy()).view(torch.float8_e4m3fn).double().numpy() * w.k_scale
    q = torch.from_numpy(w.q_bits[b, i].copy().view(np.int16)).view(torch.bfloat16).double().numpy()
    z = (q @ k.T) / np.sqrt(512)
    gap = z[:, 0] - np.median(z[:, 1:], axis=1)
    assert np.all((gap > 7.5) & (gap < 10.5))
    p = np.exp(z - z.max(axis=1, keepdims=True))
    tail = 1 - p[:, 0] / p.sum(axis=1)
    assert np.all((tail > 0.1) & (tail < 0.35))


def test_counts_for_the_benchmark_shape():
    spec = workloads.SPECS["metric"]
    assert (spec["batch"], spec["s_q"], spec["h_q"], spec["seq_len"]) == (64, 2, 64, 8196)
    w = workloads.make("tiny", batch=1, s_q=2, h_q=64, seq_len=8196, causal=True)
    # 2 * h_q * (sk-1 + sk) * 1088 per sequence
    assert workloads.flops(w) == 2 * 64 * (8195 + 8196) * 1088
    nb = workloads.algorithmic_bytes(w)
    assert nb["kv"] == 8196 * 640 and nb["q"] == 2 * 64 * 576 * 2 and nb["out"] == 2 * 64 * 512 * 2
