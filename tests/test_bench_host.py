"""Host logic of bench.py, on the CPU: the timing statistics, the byte counts
behind GB/s, the overhead bytes, the argument checks, the gate that drops
stale traffic counters and the oracle leg's parity gate.

The algorithmic bytes are pinned to the workload table of the measurement
plan, whose figures follow the Loom Kernels benchmark page's byte count for
a decode call (K and V over the valid tokens, plus Q and O): for Hq/Hkv 32/8
and D 128 in a 16-bit dtype, 4,096 bytes per token of context and 16,384
bytes per sequence."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_sample_stats_median_min_max():
    s = bench.sample_stats([3e-3, 1e-3, 2e-3])
    assert s == {"n": 3, "median_us": 2.0, "min_us": 1.0, "max_us": 3.0}
    s = bench.sample_stats([4e-3, 1e-3, 2e-3, 3e-3])
    assert s["n"] == 4 and s["median_us"] == 2.5 and s["min_us"] == 1.0 and s["max_us"] == 4.0
    assert bench.sample_stats([5e-3])["median_us"] == 5.0


# (workload, bytes) as the measurement plan's table lists them
TABLE = [
    ("tiny", 81_920),
    ("short_B1_L16_bf16_bs16", 81_920),
    ("short_B1_L32_f16_bs32", 147_456),
    ("short_B1_L64_bf16_bs32", 278_528),
    ("short_B8_L16_f16_bs16", 655_360),
    ("short_B8_L32_bf16_bs16", 1_179_648),
    ("short_B8_L64_f16_bs32", 2_228_224),
    ("short_B32_L16_bf16_bs32", 2_621_440),
    ("short_B32_L32_f16_bs16", 4_718_592),
    ("short_B32_L64_bf16_bs16", 8_912_896),
    ("splitk_B1_L128", 540_672),
    ("splitk_B1_L256", 1_064_960),
    ("splitk_B1_L512", 2_113_536),
    ("splitk_B1_L1024", 4_210_688),
    ("splitk_B8_L128", 4_325_376),
    ("splitk_B8_L256", 8_519_680),
    ("splitk_B8_L512", 16_908_288),
    ("splitk_B8_L1024", 33_685_504),
]


@pytest.mark.parametrize("name,nbytes", TABLE)
def test_algorithmic_bytes_match_the_table(name, nbytes):
    assert bench.make_workload(name).algorithmic_bytes() == nbytes


def test_fp8_bytes_halve_the_cache_reads_only():
    # E4M3FN codes are one byte: K+V reads halve, Q and O stay 16-bit
    c = bench.make_workload("splitk_B8_L1024_fp8")
    assert c.fp8
    assert c.algorithmic_bytes() == (33_685_504 - 16_384 * 8) // 2 + 16_384 * 8


def test_overhead_bytes():
    c = bench.make_workload("splitk_B8_L1024")
    o = bench.overhead_bytes(c, 4)
    assert o["block_table"] == 4 * 8 * 64 and o["context_lens"] == 4 * 8
    # fp32 partial outputs and log-sum-exps per (sequence, query head, partition)
    assert o["split_workspace_each_way"] == 4 * 8 * 32 * 4 * (128 + 1)
    assert bench.overhead_bytes(c, 1)["split_workspace_each_way"] == 0


def _run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("args", [("--samples", "-1"), ("--steps", "0")])
def test_bad_timing_arguments_exit(args):
    r = _run_bench(*args)
    assert r.returncode == 2 and r.stdout == ""


def test_traffic_counters_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    rec = {"workload": "w", "kernel_sha": "0123456789abcdef", "traffic_bytes_per_launch": 5.0}
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0123456789abcdef")
    assert bench.load_traffic("w")["traffic_bytes_per_launch"] == 5.0
    monkeypatch.setattr(bench, "kernel_sha", lambda: "fedcba9876543210")
    assert bench.load_traffic("w") is None
    assert bench.load_traffic("absent") is None


def _bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_oracle_parity_gate_accepts_the_rounded_result_and_rejects_a_wrong_one():
    c = bench.make_workload("splitk_B1_L128")
    ref, _ = bench._oracle_call(c, 1, 2)
    ok, errs, timing = bench.oracle_parity(c, _bf16_bits(ref), 1)
    assert ok and errs["sequences_checked"] == 1 and timing["nseq"] == 1
    bad = np.array(ref, dtype=np.float64)
    bad[0, 5, 17] += 0.05 + 0.05 * abs(bad[0, 5, 17])  # beyond 1e-2 + 1e-2 |r|
    ok, errs, _ = bench.oracle_parity(c, _bf16_bits(bad), 1)
    assert not ok and errs["max_abs"] > 0.04
    nan = np.array(ref, dtype=np.float64)
    nan[0, 0, 0] = np.nan
    assert not bench.oracle_parity(c, _bf16_bits(nan), 1)[0]


def test_cpu_baseline_reports_the_median_call():
    c = bench.make_workload("tiny")
    timing = {"nseq": 1, "nthreads": 1, "used": 1, "times": [0.004, 0.001, 0.002]}
    b = bench.cpu_baseline(c, timing, min_seconds=0.0, max_calls=3)
    assert b["calls"] == 3 and b["seconds_per_call"] == 0.002
    assert b["seconds_min"] == 0.001 and b["seconds_max"] == 0.004
    assert b["kind"] == "oracle" and b["unit"] == "GB/s"
    assert b["value"] == round(c.algorithmic_bytes() / 0.002 / 1e9, 4)
