"""GPU parity of per-token KV scales (one k and one v scale per cache row,
[pages, 64]) through the C ABI: the per-token quantize-on-write bit for bit,
and the decode (fp8 and bf16 dots, dense and sparse) within the dot mode's
tolerances against the oracle."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import gpu_util as gu
import workloads
from oracle import attn, cache

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _scales(w, seed, spread=8.0):
    rng = np.random.default_rng(seed)
    shape = (w.kv_cache.shape[0], 64)
    ks = (w.k_scale * rng.uniform(1.0 / spread, 1.0, shape)).astype(np.float32)
    vs = (w.v_scale * rng.uniform(1.0 / spread, 1.0, shape)).astype(np.float32)
    return ks, vs


def _decode(w, ks, vs, splits, dot="fp8"):
    t = gu.device_inputs(w)
    kst = torch.from_numpy(ks).to("cuda:0")
    vst = torch.from_numpy(vs).to("cuda:0")
    out, lse = mla.decode(t["q"], t["kv"], t["bt"], t["sl"], kst, vst, num_splits=splits, dot=dot,
                          causal=w.causal, indices=t["idx"], softmax_scale=w.softmax_scale or 0.0,
                          per_token_scales=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(w, ks, vs, splits, dot="fp8"):
    out, lse = _decode(w, ks, vs, splits, dot)
    kw = dict(d_nope=w.d_nope, d_rope=w.d_rope, causal=w.causal, softmax_scale=w.softmax_scale,
              indices=w.indices)
    ref_o, ref_l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, **kw)
    if not gu.kernel_query_exact(w, dot):
        qp = attn.dequantized_q_nope(w.q_bits)
        ref_oq, ref_lq = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs,
                                         q_nope_override=qp, **kw)
    else:
        ref_oq, ref_lq = ref_o, ref_l
    return gu.compare(out, lse, ref_o, ref_l, ref_lq, dot, ref_out_rows=ref_oq)


CASES = [
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 64, "seq_len": [700, 3], "seed": 121}),      # 4 waves, ragged
    ("tiny", {"batch": 3, "s_q": 2, "h_q": 48, "seq_len": [130, 64, 2], "seed": 122}),  # 96 rows
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 32, "seq_len": [257, 90], "seed": 123}),     # 2 waves
    ("tiny", {"batch": 2, "s_q": 1, "h_q": 16, "seq_len": [200, 33], "seed": 124}),     # 1 wave
    ("tiny", {"batch": 2, "s_q": 2, "h_q": 64, "d_rope": 0, "seq_len": [300, 64], "seed": 125}),
    ("sparse", {"batch": 2, "seq_len": 3000, "topk": 200, "seed": 128}),                # sparse gather
]

# The sparse workload is peaky: one key ~9 above the rest, whose tail holds a
# fifth of the weight at p ~ e^-9 of the top key. With per-token scales, P is
# multiplied by v_j / V_ref (<= 1) before its e4m3fn packing, which pushes
# that tail further into the format's subnormal range; the small sparse cases
# spread the scales 2x, the full configuration is run at 2x and at the dense
# cases' 8x.
SPREAD = {"tiny": 8.0, "sparse": 2.0}


@pytest.mark.parametrize("name,kw", CASES)
@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_per_token_decode_matches_oracle(name, kw, splits, dot):
    w = workloads.make(name, **kw)
    ks, vs = _scales(w, kw["seed"], SPREAD[name])
    res = _check(w, ks, vs, splits, dot)
    print(f"per-token {dot} {kw} splits={splits}: {res}")


@pytest.mark.parametrize("factor", [1e-4, 1e4, 1e6])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_per_token_decode_at_extreme_value_scales(factor, splits, dot):
    """The v-scales far from 1: the output is factor times the unscaled one,
    so every relative error must stay where it is. Split partials hold values
    over a per-row scale, which keeps them inside fp16's normal range (at
    1e-4 the values are ~1e-5, fp16 subnormals if stored as they are; at 1e6
    they pass fp16's largest value)."""
    w = workloads.make("tiny", batch=2, s_q=2, h_q=64, seq_len=[700, 190], seed=131)
    ks, vs = _scales(w, 131)
    vs = (vs.astype(np.float64) * factor).astype(np.float32)
    res = _check(w, ks, vs, splits, dot)
    print(f"per-token {dot} v-scales x{factor:g} splits={splits}: {res}")


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_per_token_decode_sparse_configuration(dot):
    w = workloads.make("sparse")
    ks, vs = _scales(w, 129, SPREAD["sparse"])
    res = _check(w, ks, vs, 0, dot)
    print(f"per-token sparse {dot}: {res}")


def test_per_token_decode_sparse_configuration_full_spread():
    w = workloads.make("sparse")
    ks, vs = _scales(w, 129, 8.0)
    res = _check(w, ks, vs, 0, "fp8")
    print(f"per-token sparse fp8, 8x spread: {res}")


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_per_token_decode_benchmark_shape(dot):
    w = workloads.make("metric")
    ks, vs = _scales(w, 126)
    res = _check(w, ks, vs, 0, dot)
    print(f"per-token metric {dot}: {res}")


def test_per_token_quantize_then_decode():
    rng = np.random.default_rng(127)
    b, s_q, h_q, sk = 3, 2, 64, 600
    ppseq = (sk + 63) // 64
    pages = b * ppseq + 2
    perm = rng.permutation(pages)[: b * ppseq].reshape(b, ppseq).astype(np.int32)
    n = b * sk
    # row magnitudes spread 4x, so the per-token scales differ (a wider spread
    # makes the logits of the largest rows dominate, and the fp8 query's own
    # rounding, not the scales, then sets the error)
    x = rng.standard_normal((n, 512)) * rng.uniform(0.5, 2.0, (n, 1))
    ckv = _bf16_bits(x)
    rope = _bf16_bits(rng.standard_normal((n, 64)))
    pos = np.arange(sk)
    slots = np.concatenate([perm[s, pos // 64] * 64 + pos % 64 for s in range(b)]).astype(np.int32)
    kv0 = np.full((pages, 64, 1, 640), 0xFF, dtype=np.uint8)
    sc0 = np.zeros((pages, 64), dtype=np.float32)
    ref_cache, ref_sc = cache.quantize_kv_per_token(ckv, rope, slots, kv0, sc0)
    dev = "cuda:0"
    kv = torch.from_numpy(kv0).to(dev)
    ks = torch.from_numpy(sc0).to(dev)
    vs = torch.from_numpy(sc0).to(dev)
    mla.quantize_kv(torch.from_numpy(ckv.view(np.int16)).view(torch.bfloat16).to(dev),
                    torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).to(dev),
                    torch.from_numpy(slots).to(dev), kv, ks, vs, compute_scale="per_token")
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), ref_cache)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), ref_sc.view(np.uint32))
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), ref_sc.view(np.uint32))
    q_bits = _bf16_bits(rng.standard_normal((b, s_q, h_q, 576)))
    w = workloads.Workload(**{**workloads.make("tiny").__dict__, "batch": b, "s_q": s_q, "h_q": h_q,
                              "q_bits": q_bits, "kv_cache": ref_cache.reshape(pages, 64, 640),
                              "block_table": perm, "seq_lens": np.full(b, sk, dtype=np.int32),
                              "indices": None, "causal": True})
    res = _check(w, ref_sc, ref_sc, 0)
    print(f"per-token quantize -> decode: {res}")
