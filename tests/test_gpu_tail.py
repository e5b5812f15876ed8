"""The pages' softmax-tail case through the HIP decode (ROCm/aiter PR #6199,
Results, accuracy paragraph, and the 'keep the softmax tail' test commit): one
key scoring 9 above 2047 keys at 0, whose tail carries about a fifth of the
output, split-K off. The fixture in tests/golden/softmax_tail.json holds the
page's figures; the oracle's closed form for this case is pinned on the CPU
(test_oracle_attn.test_softmax_tail_fixture). Every logit here is exact in
both dot modes (the query quantizes to 256 * 2^-7 without error), so the only
rounding on the fp8-dot path is that of P."""

import json
import math
import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
from oracle import attn, fp8

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "softmax_tail.json")


def _tail_case():
    g = json.load(open(GOLDEN))
    n = g["tail_keys"] + 1
    codes = np.zeros((n, 512), dtype=np.uint8)
    codes[0, 0] = 0x49                          # 4.5 on a coordinate only the first key has
    codes[1:, 1] = 0x38                         # the tail's value: 1.0 in dim 1
    codes[0, 2] = 0x38                          # the dominant key's value: 1.0 in dim 2
    pages = n // 64
    order = np.random.default_rng(2).permutation(pages + 1)
    cache = np.full((pages + 1, 64, 1, 512), 0xFF, dtype=np.uint8)
    bt = order[:pages].astype(np.int32)[None, :]
    for j in range(n):
        cache[bt[0, j // 64], j % 64, 0] = codes[j]
    q = np.zeros((1, 1, 1, 512), dtype=np.uint16)
    q[..., 0] = fp8.f32_to_bf16_bits(np.float32(2.0))   # 2.0 * 4.5 = 9 exactly
    return g, q, cache, bt, np.array([n], dtype=np.int32)


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_softmax_tail_through_the_kernel(dot):
    g, q, cache, bt, sl = _tail_case()
    ref_o, ref_l = attn.mla_decode(q, cache[:, :, 0], bt, sl, 1.0, 1.0, d_rope=0, causal=False, softmax_scale=1.0)
    dev = "cuda:0"
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    out, lse = mla.decode(qd, torch.from_numpy(cache).to(dev), torch.from_numpy(bt).to(dev),
                          torch.from_numpy(sl).to(dev), one, one, num_splits=1, dot=dot, causal=False,
                          softmax_scale=1.0)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()[0, 0, 0].astype(np.float64)
    r = ref_o[0, 0, 0]
    nz = r != 0
    max_rel = float(np.max(np.abs(o[nz] - r[nz]) / np.abs(r[nz])))
    rel_l2 = float(np.linalg.norm(o - r) / np.linalg.norm(r))
    assert np.all(o[~nz] == 0)
    print(f"softmax tail, {dot} dots: max-rel {max_rel:.4f} (page, fp8 dots with the P scale: "
          f"{g['page_fp8_dot_errors']['scaled_max_rel']}), rel-L2 {rel_l2:.4f}, "
          f"|dlse| {abs(lse.item() - ref_l[0, 0, 0]):.2e}")
    # the page's scaled fp8-dot figure is 1.8% max-rel; bf16 dots round P and
    # the output to bf16 only
    assert max_rel <= (0.025 if dot == "fp8" else 0.005)
    assert abs(lse.item() - ref_l[0, 0, 0]) <= 1e-3
    assert abs(ref_l[0, 0, 0] - 9.22524) < 1e-5 and math.isclose(r[1], 0.20167, abs_tol=1e-5)
