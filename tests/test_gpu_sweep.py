"""Seeded sweep of small decode configurations through the C ABI against the
oracle, to the usual tolerances (gpu_util.compare).

Each case draws, from one fixed generator, a combination of the options the
other tests mostly vary one at a time: dense or sparse key streams, fp8 or
bf16 dots, per-tensor or per-token scales, e4m3fn or e4m3fnuz codes (per
tensor only), with or without the 64 rope dims, causal or not, ragged and
empty sequences of up to 4000 keys (dense), contexts of up to 20000 keys and
index lists longer than the context (sparse: the tail entries are -1), 16 to
128 heads, row counts that are not multiples of 32 and more than one 128-row
group, and a split count of 1, 2, 3, 7 or automatic.
"""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import gpu_util as gu
import workloads
from oracle import attn

pytestmark = pytest.mark.gpu


def _cases(n=128, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        sparse = bool(rng.random() < 0.35)
        dot = "fp8" if rng.random() < 0.6 else "bf16"
        per_token = bool(rng.random() < 0.3)
        fnuz = (not per_token) and bool(rng.random() < 0.2)
        d_rope = 64 if rng.random() < 0.7 else 0
        splits = int(rng.choice([1, 2, 3, 7, 0]))
        kw = {"seed": 1000 + c, "d_rope": d_rope}
        if sparse:
            b = int(rng.integers(1, 4))
            kw.update(batch=b, s_q=int(rng.integers(1, 4)), h_q=int(rng.choice([16, 32, 64, 128])),
                      topk=int(rng.choice([64, 100, 257])), peaky=bool(rng.random() < 0.5),
                      seq_len=[int(x) for x in rng.integers(40, 1500 if rng.random() < 0.7 else 20000, size=b)])
            name = "sparse"
        else:
            b = int(rng.integers(1, 4))
            hi = 4000 if rng.random() < 0.2 else 900
            lens = [int(x) for x in rng.integers(0, hi, size=b)]
            if rng.random() < 0.3:
                lens[int(rng.integers(0, b))] = int(rng.choice([0, 1, 63, 64, 65]))
            kw.update(batch=b, s_q=int(rng.integers(1, 9)), h_q=int(rng.choice([16, 24, 48, 64, 128])),
                      seq_len=lens, causal=bool(rng.random() < 0.7))
            name = "tiny"
        if fnuz:
            kw["encoding"] = "e4m3fnuz"
        out.append((name, kw, dot, per_token, splits))
    return out


CASES = _cases()


def _scales(w, seed, spread):
    rng = np.random.default_rng(seed)
    shape = (w.kv_cache.shape[0], 64)
    ks = (w.k_scale * rng.uniform(1.0 / spread, 1.0, shape)).astype(np.float32)
    vs = (w.v_scale * rng.uniform(1.0 / spread, 1.0, shape)).astype(np.float32)
    return ks, vs


def _id(case):
    name, kw, dot, per_token, splits = case
    rows = kw["h_q"] if name == "sparse" else kw["s_q"] * kw["h_q"]
    return (f"{kw['seed']}-{name}-{dot}-{'tok' if per_token else 'ten'}-{kw.get('encoding', 'fn')}"
            f"-r{kw['d_rope']}-rows{rows}-s{splits}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_sweep_matches_oracle(case):
    name, kw, dot, per_token, splits = case
    w = workloads.make(name, **kw)
    t = gu.device_inputs(w)
    ka = dict(d_nope=w.d_nope, d_rope=w.d_rope, causal=w.causal, softmax_scale=w.softmax_scale,
              indices=w.indices, encoding=w.encoding)
    if per_token:
        # the peaky sparse tail sits near e4m3fn's subnormals: spread 2x there
        ks, vs = _scales(w, kw["seed"], 2.0 if (name == "sparse" and kw.get("peaky")) else 8.0)
        kst = torch.from_numpy(ks).to("cuda:0")
        vst = torch.from_numpy(vs).to("cuda:0")
    else:
        ks, vs = w.k_scale, w.v_scale
        kst, vst = t["ks"], t["vs"]
    print(f"[sweep] {_id(case)} {kw}", flush=True)
    out, lse = mla.decode(t["q"], t["kv"], t["bt"], t["sl"], kst, vst, num_splits=splits, dot=dot,
                          causal=w.causal, indices=t["idx"], softmax_scale=w.softmax_scale or 0.0,
                          per_token_scales=per_token)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs, **ka)
    if not gu.kernel_query_exact(w, dot):
        qp = attn.dequantized_q_nope(w.q_bits, w.d_nope)
        ref_oq, ref_lq = attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, ks, vs,
                                         q_nope_override=qp, **ka)
    else:
        ref_oq, ref_lq = ref_o, ref_l
    res = gu.compare(out, lse, ref_o, ref_l, ref_lq, dot, ref_out_rows=ref_oq)
    print(f"[sweep] {_id(case)}: rel {res['rel_l2']:.2e} row {res['row_rel_l2_max']:.2e} "
          f"lse {res['lse_max_abs']:.2e}", flush=True)
