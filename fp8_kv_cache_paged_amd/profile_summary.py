"""Summarize rocprofv3 outputs of a bench.py run into a short text report.

usage:
  python -m fp8_kv_cache_paged_amd.profile_summary --stats DIR --fetch DIR --write DIR \
      [--bench-json FILE] --command CMD ... --out profiles/<name>.txt

DIR are rocprofv3 output directories (``-d DIR -o NAME --output-format csv``)
of the same bench.py command: one ``--kernel-trace --stats`` run and two
``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE), plus optionally (``--util DIR``)
a ``--pmc`` run of the matrix-core and LDS counters (MfmaUtil, LdsUtil,
LDSBankConflict, LdsBankConflict, SQ_INSTS_VALU_MFMA_MOPS_F8/_BF16).

The HBM traffic of the split kernel is the per-dispatch counter value scaled
by what the same counter reads for kernels of known size in the same run: the
2 GiB streaming read that bench.py times (FETCH_SIZE) and torch's 2 GiB fill
before it (WRITE_SIZE). The report records the SHA-256 of the kernel source it
was taken with (mla_decode_ws.hip, mla_decode.hip, mla_device.h); bench.py
only reports the traffic while those are unchanged.

``--per-config NAME=DIR ... --out FILE`` instead summarizes one
``--kernel-trace --stats`` run per workload: the average duration of the
split kernel and of the combine kernel of each; ``--per-config-counters
NAME=UTIL:FETCH:WRITE ...`` adds the split kernel's utilization counters and
HBM bytes of the three --pmc runs of a workload.
"""

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# the decode kernels' sources: the report is valid while they are unchanged
KERNEL_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("mla_decode_ws.hip", "mla_decode.hip", "mla_device.h")]
SPLIT_KERNEL = "mla::mla_decode_ws_kernel<"   # the benchmark shape's split kernel (fp8 dots)
STREAM_BYTES = 2 << 30          # bench.py's HBM read probe
FILL_BYTES = 2 << 30            # torch fill of the same buffer


def source_sha256(paths=None):
    h = hashlib.sha256()
    for path in paths or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _one(pattern):
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(stats_dir):
    rows = list(csv.DictReader(open(_one(os.path.join(stats_dir, "**", "*kernel_stats.csv")))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["Percentage"])) for r in rows]


def counter_by_kernel(pmc_dir, counter):
    out = {}
    for r in csv.DictReader(open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv")))):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _match(d, needle):
    vals = [v for k, vs in d.items() if needle in k for v in vs]
    if not vals:
        raise KeyError(needle)
    return vals


def traffic(fetch_dir, write_dir, kernel=SPLIT_KERNEL):
    f = counter_by_kernel(fetch_dir, "FETCH_SIZE")
    w = counter_by_kernel(write_dir, "WRITE_SIZE")
    f_probe = _match(f, "stream_read_kernel")
    fetch_scale = STREAM_BYTES / (sum(f_probe) / len(f_probe) * 1024.0)
    w_fill = _match(w, "FillFunctor<unsigned char>")
    write_scale = FILL_BYTES / (sum(w_fill) * 1024.0)   # one fill, split over launches
    fk = _match(f, kernel)
    wk = _match(w, kernel)
    fetch_b = sum(fk) / len(fk) * 1024.0 * fetch_scale
    write_b = sum(wk) / len(wk) * 1024.0 * write_scale
    return {"fetch_scale": fetch_scale, "write_scale": write_scale, "fetch_bytes": fetch_b,
            "write_bytes": write_b, "traffic_bytes": fetch_b + write_b, "dispatches": len(fk)}


UTIL_COUNTERS = ["MfmaUtil", "LdsUtil", "LDSBankConflict", "LdsBankConflict",
                 "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_BF16"]


def utilization(util_dir, kernel=SPLIT_KERNEL):
    """Per-dispatch averages of the utilization counters for the split kernel."""
    out = {}
    for c in UTIL_COUNTERS:
        try:
            v = _match(counter_by_kernel(util_dir, c), kernel)
        except KeyError:
            continue
        out[c] = (sum(v) / len(v), len(v))
    return out


def per_config_counters(triples):
    """Lines for --pmc runs per workload: NAME=UTILDIR:FETCHDIR:WRITEDIR."""
    lines = ["", "split kernel counters per workload (--pmc runs of the same bench.py commands, per dispatch;",
             "HBM bytes scaled as in the benchmark profile):",
             f"  {'workload':<10} {'MfmaUtil%':>9} {'LdsUtil%':>8} {'LDSBankConfl%':>13} {'fetch MB':>9} {'write MB':>9}"]
    any_split = "mla::mla_decode"   # the dv-split or the row-block kernel
    for t in triples:
        name, dirs = t.split("=", 1)
        ud, fd, wd = dirs.split(":")
        ut = utilization(ud, any_split)
        tr = traffic(fd, wd, any_split)
        lines.append(f"  {name:<10} {ut['MfmaUtil'][0]:>9.1f} {ut['LdsUtil'][0]:>8.1f} "
                     f"{ut['LDSBankConflict'][0]:>13.2f} {tr['fetch_bytes'] / 1e6:>9.1f} {tr['write_bytes'] / 1e6:>9.1f}")
    return lines


def per_config(pairs, out_path, commands, counters=None):
    lines = ["# rocprofv3 kernel durations per workload (--kernel-trace --stats)", ""]
    lines += ["commands (run from /tmp with TMPDIR=/tmp; repository at /root/repo):"]
    lines += [f"  {c}" for c in commands]
    lines += ["", f"source_sha256: {source_sha256()}", "",
              f"  {'workload':<14} {'split kernel us':>16} {'calls':>6} {'combine us':>11} {'calls':>6}  split kernel"]
    for pair in pairs:
        name, d = pair.split("=", 1)
        st = kernel_stats(d)
        sk = [(c, a, n.split("<")[0].replace("void mla::", "")) for n, c, a, _ in st
              if n.startswith("void mla::mla_decode")]
        ck = [(c, a) for n, c, a, _ in st if "mla_combine_kernel" in n]
        s_c, s_a, s_n = max(sk) if sk else (0, 0.0, "-")
        c_c, c_a = max(ck) if ck else (0, 0.0)
        lines.append(f"  {name:<14} {s_a / 1e3:>16.2f} {s_c:>6} {c_a / 1e3:>11.2f} {c_c:>6}  {s_n}")
    if counters:
        lines += per_config_counters(counters)
    os.makedirs(os.path.dirname(os.path.abspath(out_path)), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--util")
    ap.add_argument("--per-config", nargs="+", default=None, metavar="NAME=DIR")
    ap.add_argument("--per-config-counters", nargs="+", default=None, metavar="NAME=UTIL:FETCH:WRITE")
    ap.add_argument("--bench-json")
    ap.add_argument("--command", action="append", default=[], help="command lines that produced DIRs")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.per_config:
        per_config(a.per_config, a.out, a.command, a.per_config_counters)
        return
    st = kernel_stats(a.stats)
    tr = traffic(a.fetch, a.write)
    lines = ["# rocprofv3 summary: mla_decode_ws_kernel (fp8 dots), benchmark workload", ""]
    lines += ["commands (run from /tmp with TMPDIR=/tmp; repository at /root/repo):"]
    lines += [f"  {c}" for c in a.command]
    lines += ["", f"source_sha256: {source_sha256()}", ""]
    lines += ["kernel stats (--kernel-trace --stats):", f"  {'calls':>6} {'avg_us':>10} {'pct':>6}  name"]
    for name, calls, avg, pct in st[:8]:
        lines.append(f"  {calls:>6} {avg / 1e3:>10.2f} {pct:>6.2f}  {name[:110]}")
    lines += ["", "HBM traffic of the split kernel (--pmc FETCH_SIZE / WRITE_SIZE, per dispatch):",
              f"  FETCH_SIZE scale {tr['fetch_scale']:.4f} (2 GiB streaming read), "
              f"WRITE_SIZE scale {tr['write_scale']:.4f} (2 GiB fill)",
              f"  fetch_bytes_per_launch: {tr['fetch_bytes']:.0f}",
              f"  write_bytes_per_launch: {tr['write_bytes']:.0f}",
              f"traffic_bytes_per_launch: {tr['traffic_bytes']:.0f}",
              f"  dispatches averaged: {tr['dispatches']}"]
    if a.util:
        ut = utilization(a.util)
        lines += ["", "matrix-core and LDS counters of the split kernel (--pmc, per dispatch):"]
        for c, (v, nd) in ut.items():
            lines.append(f"  {c}: {v:.4g}  ({nd} dispatches)")
        if "SQ_INSTS_VALU_MFMA_MOPS_F8" in ut:
            lines.append(f"  fp8 MFMA flops per dispatch (MOPS_F8 x 512): {ut['SQ_INSTS_VALU_MFMA_MOPS_F8'][0] * 512:.4g}")
    if a.bench_json:
        rec = [json.loads(l) for l in open(a.bench_json) if l.strip().startswith("{")][-1]
        rf = rec.get("roofline", {})
        lines += ["", "bench.py line of the --kernel-trace run:",
                  f"  ms_per_call {rec.get('ms_per_step')}, split kernel (HIP events) {rf.get('kernel_us')} us, "
                  f"algorithmic bytes/launch {rf.get('bytes_per_launch')}, achieved {rf.get('achieved')} GB/s"]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
