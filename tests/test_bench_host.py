"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes and flops every rate is divided by, counted here by hand for small
cases; the percentile summary of a kernel trace; the refusal of a
multi-GPU run."""

import csv
import json
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import make_case, make_config_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_tiny_workload_by_hand():
    # one sequence of 256 tokens (4 pages), one query token, 16 heads
    case = make_config_case(1)
    nb, fl = bench.algorithmic_work(case)
    rows = 16
    kv = 256 * 576 * 2              # every cached latent read once
    q = rows * 576 * 2              # absorbed query rows in
    out = rows * 512 * 2 + rows * 4  # bf16 output rows and fp32 lse out
    tables = 4 * 4 + 4              # four block-table entries and one length
    assert nb == kv + q + out + tables
    assert fl == 2 * (576 + 512) * rows * 256


def test_algorithmic_work_counts_causal_visibility():
    # s_q = 2, causal: query token i of a sequence of L sees L - 1 + i tokens;
    # an empty sequence contributes no flops and no cache bytes
    case = make_case([100, 1, 0], 2, 4, True, seed=3)
    nb, fl = bench.algorithmic_work(case)
    vis = (99 + 100) + (0 + 1) + 0
    assert fl == 2 * (576 + 512) * 4 * vis
    rows = 2 * 4
    pages = 2 + 1 + 0
    expect = (1152 * 101 + 3 * rows * (1152 + 1024 + 4) + 4 * pages + 4 * 3)
    assert nb == expect


def test_algorithmic_work_non_causal_ignores_s_q_offset():
    case = make_case([70], 3, 2, False, seed=4)
    _, fl = bench.algorithmic_work(case)
    assert fl == 2 * (576 + 512) * 2 * 3 * 70


def test_percentiles_of_a_trace(tmp_path, capsys):
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, d in enumerate([10, 20, 30, 40, 50]):  # microseconds
            w.writerow(["decode", 1_000_000 * i, 1_000_000 * i + 1000 * d])
        w.writerow(["combine", 0, 4000])
    bench.trace_stats(str(path))
    out = json.loads(capsys.readouterr().out)
    dec = out["decode"]
    assert dec["n"] == 5 and dec["mean"] == 30.0 and dec["p50"] == 30.0
    assert np.isclose(dec["p10"], 14.0) and np.isclose(dec["p90"], 46.0)
    assert out["combine"]["mean"] == 4.0


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
