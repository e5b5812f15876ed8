"""The role-split kernel's two-term forms (at most 16 query rows per key
stream): the second terms of the query (both dot modes) and of P (bf16 dots)
ride in columns 16..31 of the one row block, and both column halves must take
their row's own causal limit, the row being column % 16.

Checked against the plain oracle (the kernel multiplies the exact bf16 query
here), at the dot mode's tolerances: row counts that mix several query tokens
in the 16 columns (s_q * h_q = 16 with s_q = 2, 4, 16; fewer rows), causal
rows whose visible lengths differ, and query rows whose values span many
binades (the second term is exact for every element of at least 2^-6 of the
row's scale).
"""

import numpy as np
import pytest

import gpu_util as gu
import workloads

pytestmark = pytest.mark.gpu

SHAPES = [
    {"batch": 2, "s_q": 2, "h_q": 8, "seq_len": [300, 70]},     # two tokens of 8 heads
    {"batch": 2, "s_q": 4, "h_q": 4, "seq_len": [129, 3]},      # four tokens, one sequence shorter than s_q
    {"batch": 1, "s_q": 16, "h_q": 1, "seq_len": [200]},        # sixteen tokens of one head
    {"batch": 3, "s_q": 3, "h_q": 1, "seq_len": [64, 65, 1]},   # three rows
    {"batch": 2, "s_q": 1, "h_q": 16, "d_rope": 0, "seq_len": [500, 17]},
]


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_two_term_rows_match_the_plain_oracle(idx, splits, dot):
    kw = dict(SHAPES[idx])
    w = workloads.make("tiny", seed=300 + idx, causal=True, **kw)
    assert gu.kernel_query_exact(w, dot)
    res = gu.check(w, gu.OracleCache(w), dot, num_splits=splits)
    assert res["lse_max_abs_vs_bf16q"] <= gu.LSE_TOL
    print(f"two-term {kw} splits={splits} dot={dot}: {res}")


@pytest.mark.parametrize("dot", ["fp8", "bf16"])
def test_two_term_query_over_many_binades(dot):
    """Each query row's nope values are scaled by powers of two from 2^-20 to
    2^6 (in blocks of 32 dims), so that the row's exponent is set by the
    largest block and the smallest sit far below it: the two-term query is
    exact down to 2^-6 of the row's scale and the rest is rounded on
    e4m3fn's subnormal grid, 2^-9 of the scale at most."""
    w = workloads.make("tiny", seed=321, batch=2, s_q=2, h_q=8, seq_len=[400, 150], causal=True)
    q = w.q_bits.view(np.uint16).astype(np.uint32) << 16
    qf = q.view(np.float32).reshape(w.q_bits.shape).astype(np.float64)
    scale = 2.0 ** np.repeat(np.linspace(-20, 6, 16).round(), 32)
    qf[..., :512] *= scale
    # back to bf16 bits (round to nearest even through torch's cast)
    import torch
    w.q_bits = torch.from_numpy(qf.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    res = gu.check(w, gu.OracleCache(w), dot, num_splits=0)
    assert res["lse_max_abs_vs_bf16q"] <= gu.LSE_TOL
    print(f"two-term, query over many binades, {dot} dots: {res}")
