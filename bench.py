#!/usr/bin/env python3
"""Benchmark of the FP8-KV paged MLA decode on one MI355X.

Default workload: the benchmark shape b=64, s_q=2 (causal), h_q=64, sk=8196,
d=576 (512 e4m3fn + 64 bf16 rope), dv=512, 64-token shuffled pages, fp8 dots,
auto splits. A step is one whole decode call (split kernel + combine) over one
batch. Calls rotate through enough copies of the KV pool (>= 1 GiB together)
that the 256 MiB Infinity Cache cannot serve them, so every call reads HBM.

Prints one JSON line: throughput in TFLOP/s (useful FLOPs 2*rows*keys*(576+512)),
plus ms/call, algorithmic HBM GB/s, a roofline object for the dominant kernel
(its launches timed with HIP events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_kv_cache_paged_amd as mla  # noqa: E402
import workloads  # noqa: E402

METRIC = "FP8-KV MLA decode ms, TFLOPS, HBM GB/s (b=64, s_q=2, sk=8196, h_q=64)"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0


def split_kernel_bytes(nbytes, splits):
    """Algorithmic bytes the split kernel is responsible for: KV rows, Q and the
    tables; out and lse too when there is one split (else the combine writes them)."""
    return nbytes["kv"] + nbytes["q"] + nbytes["tables"] + (0 if splits > 1 else nbytes["out"] + nbytes["lse"])


def split_kernel_bound(flops, kern_bytes, dot):
    """The larger of the kernel's two floors: its bytes at the HBM peak, or the
    call's FLOPs at the dot type's MFMA peak."""
    mfma_peak = FP8_PEAK_TFLOPS if dot == "fp8" else BF16_PEAK_TFLOPS
    return "mfma" if flops / (mfma_peak * 1e12) > kern_bytes / (HBM_PEAK_GBPS * 1e9) else "hbm"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # (a call takes ~0.1 ms; the hardware probes run after the timed regions)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="metric", choices=sorted(workloads.SPECS))
    ap.add_argument("--dot", default="fp8", choices=["fp8", "bf16"])
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic")
    ap.add_argument("--rotate-bytes", type=float, default=1.0, help="GiB of KV copies to rotate through")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scales", default="tensor", choices=["tensor", "token"],
                    help="per-tensor k/v scales, or one per cache row (fp8 dots, dense)")
    ap.add_argument("--kv-encoding", default="e4m3fn", choices=["e4m3fn", "e4m3fnuz"],
                    help="the cache's one-byte code (gfx942's e4m3fnuz: bf16 dots, per-tensor scales)")
    ap.add_argument("--op", default="decode", choices=["decode", "quantize"],
                    help="decode (the benchmark) or the quantize-on-write of the benchmark's cache")
    return ap.parse_args()


def hbm_read_probe(dev, gib=2.0, reps=5):
    """Measured HBM read bandwidth (GB/s) of a plain streaming read kernel."""
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(1 << 16, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    mla.stream_read(src, sink)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        mla.stream_read(src, sink)
        e1.record(stream)
        e1.synchronize()
        best = max(best, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src
    torch.cuda.empty_cache()
    return best


def mfma_probe(dev, dot, reps=3):
    """Measured matrix-core throughput (TFLOP/s) with no memory traffic."""
    blocks, iters = 4096, (2048 if dot == "fp8" else 4096)   # ~3.5 ms per launch
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    mla.mfma_probe(dot, iters, blocks, sink)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flop = mla.mfma_probe(dot, iters, blocks, sink)
        e1.record(stream)
        e1.synchronize()
        best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


PROFILE = os.path.join(ROOT, "profiles", "mla_decode_ws_kernel.benchmark_workload.txt")


def measured_traffic():
    """HBM bytes per split-kernel launch from the committed rocprofv3 counter
    summary, or None when it was taken on another version of the kernel."""
    from fp8_kv_cache_paged_amd import profile_summary
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    fields = dict(l.strip().split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith(" "))
    if fields.get("source_sha256") != profile_summary.source_sha256():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s):
    """The oracle (float64 NumPy, unmodified) on a bounded sample of sequences."""
    from oracle import attn
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    flops_done, t_used, seqs = 0.0, 0.0, 0
    per_seq_flops = []
    for b in range(w.batch):
        sub = workloads.Workload(**{**w.__dict__, "batch": 1, "q_bits": w.q_bits[b:b + 1],
                                    "block_table": w.block_table[b:b + 1], "seq_lens": w.seq_lens[b:b + 1],
                                    "indices": None if w.indices is None else w.indices[b:b + 1]})
        t0 = time.perf_counter()
        attn.mla_decode(sub.q_bits, sub.kv_cache, sub.block_table, sub.seq_lens, sub.k_scale, sub.v_scale,
                        d_nope=sub.d_nope, d_rope=sub.d_rope, causal=sub.causal, indices=sub.indices,
                        softmax_scale=sub.softmax_scale, encoding=sub.encoding)
        t_used += time.perf_counter() - t0
        flops_done += workloads.flops(sub)
        seqs += 1
        if t_used >= budget_s:
            break
    tflops = flops_done / t_used / 1e12
    sec_per_call = t_used * (workloads.flops(w) / flops_done)
    return {"value": tflops, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{seqs} of {w.batch} sequences of the same workload ({t_used:.1f} s); "
                      f"scaled: {sec_per_call:.2f} s per full call"}


def main_quantize(args, dev):
    """Quantize-on-write of the benchmark shape's whole cache in one call: 64
    sequences x 8196 tokens of bf16 latent (512) + rope (64) into shuffled
    64-token pages, the scale computed (amax / 448). Algorithmic bytes per
    token: 1152 read + 4 (slot) + 640 written."""
    b, sk = 64, 8196
    ppseq = (sk + 63) // 64
    pages = b * ppseq
    n = b * sk
    g = torch.Generator(device="cpu").manual_seed(6)
    ckv = torch.randn((n, 512), generator=g).to(torch.bfloat16).to(dev)
    rope = torch.randn((n, 64), generator=g).to(torch.bfloat16).to(dev)
    perm = torch.randperm(pages, generator=g).to(torch.int64)
    pos = torch.arange(sk)
    slots = torch.cat([perm[s * ppseq + pos // 64] * 64 + pos % 64 for s in range(b)]).to(torch.int32).to(dev)
    kv = torch.full((pages, 64, 1, 640), 0xFF, dtype=torch.uint8, device=dev)
    ks = torch.zeros(1, dtype=torch.float32, device=dev)
    vs = torch.zeros(1, dtype=torch.float32, device=dev)
    ws = torch.empty(mla.lib().mla_fp8_quantize_kv_workspace_size(), dtype=torch.uint8, device=dev)
    mla.quantize_kv(ckv, rope, slots, kv, ks, vs, workspace=ws)
    import ctypes
    L = mla.lib()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    stream = torch.cuda.current_stream()

    def timed(mode):
        a = (n, 64, pages, vp(ckv), vp(rope), vp(slots), vp(kv), vp(ks), vp(vs), mode, vp(ws), ws.numel(), st)
        for _ in range(args.warmup):
            L.mla_fp8_quantize_kv(*a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            rc = L.mla_fp8_quantize_kv(*a)
            if rc != 0:
                raise RuntimeError(mla.status_string(rc))
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = timed(1)          # scale computed: the amax pass, then the encode pass
    ms_given = timed(0)    # scale given: the encode pass alone
    nbytes = n * (1152 + 4 + 640)
    # the amax pass reads every written row's 512 nope values (and its slot)
    # again before the encode pass reads and writes them: 1.57x the
    # algorithmic bytes when the scale is computed, 1.0x when it is given
    moved = nbytes + n * (1024 + 4)
    gbps = nbytes / (ms * 1e-3) / 1e9
    hbm_meas = hbm_read_probe(dev)   # after the timed regions, as for the decode
    line = {
        "metric": "FP8 KV quantize-on-write GB/s (64 x 8196 tokens, 576-wide latent)",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->fp8", "data": "synthetic",
        "config": {"workload": f"quantize: {n} tokens, {pages} shuffled pages, scale computed"},
        "hbm_measured_gbps": round(hbm_meas, 1), "frac_of_measured_hbm": round(gbps / hbm_meas, 4),
        "bytes_moved_per_call": moved, "moved_over_algorithmic": round(moved / nbytes, 3),
        "given_scale": {"ms_per_step": round(ms_given, 5), "gbps": round(nbytes / (ms_given * 1e-3) / 1e9, 1),
                        "frac_of_measured_hbm": round(nbytes / (ms_given * 1e-3) / 1e9 / hbm_meas, 4),
                        "moved_over_algorithmic": 1.0},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "kv_amax_kernel + kv_encode_kernel", "bytes_per_launch": nbytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import cache
        m = 16384
        c_bits = ckv[:m].view(torch.int16).cpu().numpy().view(np.uint16)
        r_bits = rope[:m].view(torch.int16).cpu().numpy().view(np.uint16)
        sl = np.arange(m, dtype=np.int32)
        cache_np = np.full(((m + 63) // 64, 64, 1, 640), 0xFF, dtype=np.uint8)
        t0 = time.perf_counter()
        cache.quantize_kv(c_bits, r_bits, sl, cache_np)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(m * (1152 + 4 + 640) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "sample": f"{m} of {n} tokens ({dt:.1f} s)"}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 (sequences shard across "
                                   "GPUs with no exchange, so N GPUs run N copies of this workload)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not mla.library_available():
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "quantize":
        return main_quantize(args, dev)

    w = workloads.make(args.workload, encoding=args.kv_encoding)
    flops = workloads.flops(w)
    nbytes = workloads.algorithmic_bytes(w)
    print(f"[bench] workload {args.workload}: b={w.batch} s_q={w.s_q} h_q={w.h_q} d_rope={w.d_rope} "
          f"topk={w.topk} kv={w.kv_cache.nbytes / 1e6:.1f} MB", file=sys.stderr, flush=True)

    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    ks = torch.tensor([w.k_scale], dtype=torch.float32, device=dev)
    vs = torch.tensor([w.v_scale], dtype=torch.float32, device=dev)
    per_token = args.scales == "token"
    if per_token:   # one scale per cache row, spread 8x below the per-tensor value
        g = torch.Generator(device="cpu").manual_seed(7)
        shape = (w.kv_cache.shape[0], 64)
        ks = (w.k_scale * (0.125 + 0.875 * torch.rand(shape, generator=g))).to(torch.float32).to(dev)
        vs = (w.v_scale * (0.125 + 0.875 * torch.rand(shape, generator=g))).to(torch.float32).to(dev)
    idx = None if w.indices is None else torch.from_numpy(w.indices).to(dev)
    kv0 = torch.from_numpy(w.kv_cache).to(dev)
    copies = max(1, int(np.ceil(args.rotate_bytes * (1 << 30) / kv0.numel())))
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    if args.kv_encoding == "e4m3fnuz":   # the library reads the encoding from the tensor's dtype
        kvs = [k.view(torch.float8_e4m3fnuz) for k in kvs]
        kv0 = kvs[0]
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)
    p = mla.params_for(q, kv0, bt, causal=w.causal, dot=args.dot, indices=idx, per_token_scales=per_token)
    splits = args.splits or mla.resolve_splits(p, 0, mla.cu_count(dev))
    ws_bytes = mla.workspace_size(p, splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    # one call through the binding to validate everything, then the C entry
    # points directly with prebuilt arguments, so that host overhead stays far
    # below a kernel's duration and launches queue up back to back
    mla.decode(q, kv0, bt, sl, ks, vs, num_splits=splits, dot=args.dot, causal=w.causal, indices=idx,
               out=out, lse=lse, workspace=ws, per_token_scales=per_token)
    import ctypes
    L = mla.lib()
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    argsets = [(ctypes.byref(p), vp(q), vp(kv), vp(bt), vp(sl), vp(ks), vp(vs), splits, vp(out), vp(lse),
                vp(idx), vp(ws), ws.numel(), st) for kv in kvs]

    def call(i, partials_only=False):
        fn = L.mla_fp8_decode_partials if partials_only else L.mla_fp8_decode
        rc = fn(*argsets[i % copies])
        if rc != 0:
            raise RuntimeError(f"decode failed: {mla.status_string(rc)}")

    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    time.sleep(0.25)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()

    # whole-call timing: K steps between two events, synchronised on both sides
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        call(i)
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # the dominant (split) kernel alone, timed like the whole call: K
    # back-to-back launches between one pair of events on the launch stream,
    # after the same warm-up from the same rested state. The GPU's clocks
    # boost for the first ~20 calls after a pause, then dip for ~150 calls
    # before they settle (rocprofv3 traces: ~84, ~100-118, ~88 us for this
    # kernel at the benchmark shape), so with a short run the two regions
    # would otherwise see different clocks.
    time.sleep(0.25)
    for i in range(args.warmup):
        call(i, partials_only=True)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(args.steps):
        call(i, partials_only=True)
    k1.record(stream)
    k1.synchronize()
    kern_ms = k0.elapsed_time(k1) / args.steps
    assert torch.isfinite(out.float()).all(), "non-finite output"
    if splits == 1:
        kern_ms = min(kern_ms, ms_per_step)   # one kernel: the same launches timed twice

    # the hardware probes run after the timed regions: their ~20 ms of
    # saturating traffic lowers the clocks for hundreds of decode calls after
    hbm_meas = hbm_read_probe(dev)
    print(f"[bench] measured HBM read bandwidth {hbm_meas:.0f} GB/s", file=sys.stderr, flush=True)
    mfma_meas = mfma_probe(dev, args.dot)
    print(f"[bench] measured {args.dot} matrix-core throughput {mfma_meas:.0f} TFLOP/s", file=sys.stderr, flush=True)

    kern_bytes = split_kernel_bytes(nbytes, splits)
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbps = nbytes["total"] / (ms_per_step * 1e-3) / 1e9
    mfma_peak = FP8_PEAK_TFLOPS if args.dot == "fp8" else BF16_PEAK_TFLOPS
    # every fp8-dot decode runs the role-split kernel; bf16-dot decodes too
    # (two-term operands) with at most 16 rows per key stream and an e4m3fn
    # cache, the others the row-block kernel
    rows = w.h_q if w.topk else w.s_q * w.h_q
    if args.dot == "fp8" or (rows <= 16 and args.kv_encoding == "e4m3fn"):
        kernel_name = "mla_decode_ws_kernel"
    else:
        kernel_name = "mla_decode_rows_kernel"
    roofline = {"kernel": kernel_name, "kernel_us": round(kern_ms * 1e3, 2), "bytes_per_launch": kern_bytes,
                "flop_per_launch": flops, "timing": f"{args.steps} back-to-back launches between one event pair"}
    if kern_ms > ms_per_step * 1.02:
        print(f"[bench] warning: split kernel {kern_ms * 1e3:.1f} us > whole call {ms_per_step * 1e3:.1f} us "
              "(clock drift between the two timed regions)", file=sys.stderr, flush=True)
    # the committed counter summary covers the benchmark workload's fp8, per-tensor-scale launch only
    traffic = (measured_traffic() if (args.workload == "metric" and args.dot == "fp8" and not per_token
                                      and args.kv_encoding == "e4m3fn") else None)
    if split_kernel_bound(flops, kern_bytes, args.dot) == "mfma":
        kern_tflops = flops / (kern_ms * 1e-3) / 1e12
        roofline.update({"bound": "mfma", "achieved": round(kern_tflops, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                         "frac": round(kern_tflops / mfma_peak, 4), "traffic": traffic})
    else:
        roofline.update({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic})
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.dot == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: b={w.batch} s_q={w.s_q} h_q={w.h_q} "
                               f"sk={int(w.seq_lens.max())} d={w.d_nope + w.d_rope} dv={w.d_nope} "
                               f"page=64 {'causal' if w.causal else 'non-causal'}"
                               + (f" topk={w.topk}" if w.topk else ""),
                   "dots": args.dot, "splits": splits, "kv_copies_rotated": copies,
                   "scales": "per token" if per_token else "per tensor", "kv_encoding": args.kv_encoding},
        "ms_per_call": round(ms_per_step, 5),
        "hbm_gbps": round(gbps, 1),
        "hbm_measured_gbps": round(hbm_meas, 1),
        "frac_of_measured_hbm": round(gbps / hbm_meas, 4),
        "frac_of_mfma_peak": round(tflops / (FP8_PEAK_TFLOPS if args.dot == "fp8" else BF16_PEAK_TFLOPS), 4),
        "mfma_measured_tflops": round(mfma_meas, 1),
        "frac_of_measured_mfma": round(tflops / mfma_meas, 4),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
