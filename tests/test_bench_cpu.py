"""bench.py's host logic: the one-GPU guard and the roofline bound per workload."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.parametrize("name,dot,bound", [
    ("metric", "fp8", "hbm"),       # 413 FLOP/B against an fp8 ridge of 625
    ("metric", "bf16", "mfma"),     # the same intensity against a bf16 ridge of 312.5
    ("prefill", "fp8", "mfma"),     # each 128-row group reuses every key many times
    ("sparse", "fp8", "hbm"),
])
def test_roofline_bound(name, dot, bound):
    w = workloads.make(name)
    nbytes = workloads.algorithmic_bytes(w)
    kb = bench.split_kernel_bytes(nbytes, 4)
    assert kb == nbytes["kv"] + nbytes["q"] + nbytes["tables"]
    assert bench.split_kernel_bound(workloads.flops(w), kb, dot) == bound


def test_split_kernel_bytes_counts_the_output_with_one_split():
    nb = {"kv": 10, "q": 3, "tables": 1, "out": 5, "lse": 2}
    assert bench.split_kernel_bytes(nb, 1) == 21 and bench.split_kernel_bytes(nb, 2) == 14
