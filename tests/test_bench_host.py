"""Host-side parts of bench.py (CPU): the one-GPU refusal, the counter-summary
readers that feed the roofline's `traffic`, the merge byte count, and the
shape of the CPU-baseline record."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from document_masked_attention_amd.workloads import custom_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_use():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _summary(path, kernel_hash, **vals):
    with open(path, "w") as f:
        f.write("# header line: a comment\n")
        f.write("kernel: fwd_kernel\n")
        for k, v in vals.items():
            f.write(f"{k}: {v}\n")
        f.write(f"kernel_source_sha256_16: {kernel_hash}\n")


def test_traffic_read_only_from_a_summary_of_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.read_traffic("fwd_kernel") is None                      # no summary
    assert bench.read_traffic("not_a_kernel") is None
    cur = bench.kernel_source_hash(bench.KERNEL_SOURCES["fwd_kernel"])
    _summary(bench.pmc_file("fwd_kernel"), cur, hbm_bytes_per_launch=123456789)
    assert bench.read_traffic("fwd_kernel") == 123456789.0
    _summary(bench.pmc_file("fwd_kernel"), "0123456789abcdef", hbm_bytes_per_launch=123456789)
    assert bench.read_traffic("fwd_kernel") is None                      # taken on other source
    _summary(bench.pmc_file("fwd_kernel"), cur, hbm_bytes_per_launch="n/a")
    assert bench.read_traffic("fwd_kernel") is None


def test_merge_traffic_read_only_from_a_summary_of_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    path = os.path.join(str(tmp_path), bench.MERGE_PMC)
    cur = bench.kernel_source_hash(["merge.hip", "common.h", "kernels.h"])
    vals = {"merge_kernel.hbm_bytes_per_pass": 1000, "merge_kernel_f32.hbm_bytes_per_pass": 2000}
    _summary(path, cur, **vals)
    assert bench.read_merge_traffic("merge_kernel") == 1000.0
    assert bench.read_merge_traffic("merge_kernel_f32") == 2000.0
    _summary(path, "0123456789abcdef", **vals)
    assert bench.read_merge_traffic("merge_kernel") is None


def test_kernel_source_hash_follows_the_file_contents():
    a = bench.kernel_source_hash(["fwd.hip"])
    assert a == bench.kernel_source_hash(["fwd.hip"]) and len(a) == 16
    assert a != bench.kernel_source_hash(["bwd.hip"])
    assert bench.kernel_source_hash(["fwd.hip", "common.h"]) != a


def test_merge_bytes_hand_count():
    # 3 partials, 2 heads, 4 rows, D = 8; 5 of the 24 partial LSEs are -inf
    lse = np.zeros((3, 2, 4))
    lse[0, 0, :] = -np.inf
    lse[2, 1, 1] = -np.inf
    d = 8
    reads_lse = 3 * 2 * 4 * 4                  # every partial LSE, fp32
    reads_o = (24 - 5) * 2 * d                 # O slices of finite partials, bf16
    writes = 4 * 2 * (2 * d + 4)               # merged O (bf16) and LSE (fp32) per (row, head)
    assert bench.merge_bytes(lse, d) == reads_lse + reads_o + writes


def test_cpu_baseline_record_on_a_tiny_sample():
    w = custom_workload(7, [40, 25, 70, 300, 9], 4, 2, 32, backward=True)
    cb = bench.cpu_baseline(w, min_tokens=100, merge_rows=8)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] == len(os.sched_getaffinity(0))
    assert "first 135 tokens (3 whole documents)" in cb["sample"]
    assert cb["cpu"]
    comp = cb["components"]
    assert comp["fwd"]["unit"] == "TFLOP/s" and comp["fwd"]["value"] > 0
    assert comp["merge"]["unit"] == "GB/s" and comp["merge"]["value"] > 0
    assert comp["merge"]["bytes"] > 0
