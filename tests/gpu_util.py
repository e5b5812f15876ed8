"""Shared helpers for the GPU tests: move a workload to the device, run the
library through its C ABI, and compare with the oracle.

Tolerances (stated by the decode's specification): relative L2 error of `out`
<= 0.5% with bf16 dots and <= 5% with fp8 dots, over the rows that see at
least one key; `lse` within 1e-3 absolute on those rows; rows with no visible
key must give out == 0 exactly and lse == -inf. For fp8 dots the lse is
compared with the oracle evaluated at the kernel's quantized query Q' (the
quantization itself is checked bit-exactly elsewhere), and `out` with the
oracle at the exact bf16 query. The lse difference from the oracle at the
exact bf16 query is reported beside it (for fp8 dots it is the effect of
quantizing Q and exceeds 1e-3 on short or peaky rows). With at most 16 query
rows per key stream the kernel multiplies the exact bf16 query in both dot
modes (its second term rides in the half row block the rows leave free), and
the plain oracle is the reference for lse and rows there too
(kernel_query_exact).

Beside the whole-tensor figure every query row (b, i, h) is held to its own
relative L2 error against the oracle at the query the kernel multiplies (Q'
for fp8 dots, whose effect on a row the oracle reproduces exactly, and the
bf16 query for bf16 dots). What is left is the rounding of P and of the
output: fp8 dots round each weight to e4m3fn (3 mantissa bits: at most 2^-4
relative while normal, about 3.6% RMS), and these errors are independent
across keys and averaged over the 512 output dims, so a row's error sits near
that RMS; the bound is 2^-3 = 12.5%. bf16 dots round P and the output to bf16
(2^-9 each, about 0.16% RMS together); the bound is 1%. A zeroed, stale or
misplaced row block gives a row error near 100%.
"""

import functools

import numpy as np
import torch

import fp8_kv_cache_paged_amd as mla
from oracle import attn

OUT_TOL = {"bf16": 5e-3, "fp8": 5e-2}
ROW_TOL = {"bf16": 1e-2, "fp8": 0.125}
LSE_TOL = 1e-3


def device_inputs(w, device="cuda:0"):
    t = {
        "q": torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(device),
        # a uint8 view is read as e4m3fn; an fnuz cache goes in as torch's fnuz dtype
        "kv": (torch.from_numpy(w.kv_cache).to(device) if w.encoding == "e4m3fn"
               else torch.from_numpy(w.kv_cache).to(device).view(torch.float8_e4m3fnuz)),
        "bt": torch.from_numpy(w.block_table).to(device),
        "sl": torch.from_numpy(w.seq_lens).to(device),
        "ks": torch.tensor([w.k_scale], dtype=torch.float32, device=device),
        "vs": torch.tensor([w.v_scale], dtype=torch.float32, device=device),
        "idx": None if w.indices is None else torch.from_numpy(w.indices).to(device),
    }
    return t


def run(w, t, dot, num_splits=None, **kw):
    ns = w.num_splits if num_splits is None else num_splits
    out, lse = mla.decode(t["q"], t["kv"], t["bt"], t["sl"], t["ks"], t["vs"], num_splits=ns, dot=dot,
                          causal=w.causal, indices=t["idx"], softmax_scale=w.softmax_scale or 0.0, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def kernel_query_exact(w, dot):
    """Whether the default decode multiplies the exact bf16 query: bf16 dots,
    or at most 16 rows per key stream (the role-split kernel's two-term query;
    the variant kernels always quantize it for fp8 dots)."""
    rows = w.h_q if w.indices is not None else w.s_q * w.h_q
    return dot == "bf16" or rows <= 16


def oracle(w, q_prime=False):
    qo = attn.dequantized_q_nope(w.q_bits, w.d_nope) if q_prime else None
    return attn.mla_decode(w.q_bits, w.kv_cache, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                           d_nope=w.d_nope, d_rope=w.d_rope, causal=w.causal,
                           softmax_scale=w.softmax_scale, indices=w.indices, q_nope_override=qo,
                           encoding=w.encoding)


class OracleCache:
    """Oracle results per workload (the bf16-q and the Q' variants)."""

    def __init__(self, w):
        self.w = w

    @functools.cached_property
    def exact(self):
        return oracle(self.w, q_prime=False)

    @functools.cached_property
    def qprime(self):
        return oracle(self.w, q_prime=True)


def page_metrics(x, y, name):
    """The accuracy figures of FlashMLA PR #82's H800 test report (out and lse:
    cos_diff, RMSE, amax_diff), read as: cos_diff = 1 - cosine similarity of
    the flattened tensors, RMSE = root mean square of x - y, amax_diff =
    max |x - y|, all in float64 (the page names them without a formula)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    if x.size == 0:
        return {}
    nx, ny = np.linalg.norm(x), np.linalg.norm(y)
    cos = float(np.dot(x, y) / (nx * ny)) if nx > 0 and ny > 0 else 1.0
    d = x - y
    return {f"{name}_cos_diff": 1.0 - cos, f"{name}_rmse": float(np.sqrt(np.mean(d * d))),
            f"{name}_amax_diff": float(np.max(np.abs(d)))}


def compare(out, lse, ref_out, ref_lse, ref_lse_for_lse=None, dot="fp8", ref_out_rows=None):
    """Returns a dict of error figures and asserts the tolerances. ref_out,
    ref_lse: the oracle at the bf16 query; ref_lse_for_lse and ref_out_rows:
    the oracle at the query the kernel multiplies (Q' for fp8 dots), used for
    the lse and per-row checks (default: ref_lse, ref_out)."""
    ref_lse_l = ref_lse if ref_lse_for_lse is None else ref_lse_for_lse
    ref_rows = ref_out if ref_out_rows is None else ref_out_rows
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "rows with no visible key must give lse = -inf (and only they)"
    assert np.all(out[empty] == 0), "rows with no visible key must give out = 0"
    assert np.all(np.isfinite(out)), "non-finite output"
    live = ~empty
    num = np.linalg.norm((out - ref_out)[live])
    den = np.linalg.norm(ref_out[live])
    rel = float(num / den) if den > 0 else float(num)
    dl = float(np.max(np.abs(lse[live] - ref_lse_l[live]))) if live.any() else 0.0
    dl_plain = float(np.max(np.abs(lse[live] - ref_lse[live]))) if live.any() else 0.0
    row_err = np.linalg.norm((out - ref_rows)[live], axis=-1)
    row_ref = np.linalg.norm(ref_rows[live], axis=-1)
    row_rel = row_err / np.where(row_ref > 0, row_ref, 1.0)
    row_max = float(row_rel.max()) if row_rel.size else 0.0
    res = {"rel_l2": rel, "row_rel_l2_max": row_max, "lse_max_abs": dl, "lse_max_abs_vs_bf16q": dl_plain}
    res.update(page_metrics(out[live], ref_out[live], "out"))
    res.update(page_metrics(lse[live], ref_lse_l[live], "lse"))
    assert rel <= OUT_TOL[dot], f"rel-L2 {rel:.3e} > {OUT_TOL[dot]} ({dot} dots)"
    assert row_max <= ROW_TOL[dot], f"worst row rel-L2 {row_max:.3e} > {ROW_TOL[dot]} ({dot} dots)"
    assert dl <= LSE_TOL, f"max |dlse| {dl:.3e} > {LSE_TOL}"
    return res


def check(w, oc, dot, num_splits=None, t=None, **kw):
    t = device_inputs(w) if t is None else t
    out, lse = run(w, t, dot, num_splits, **kw)
    ref_o, ref_l = oc.exact
    ref_q = oc.exact if kernel_query_exact(w, dot) else oc.qprime
    return compare(out, lse, ref_o, ref_l, ref_q[1], dot, ref_out_rows=ref_q[0])
