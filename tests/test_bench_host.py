"""Host-side parts of bench.py that need no GPU: the one-GPU guard, the recorded-traffic
lookup keyed by the kernel sources' hash, and the oracle's CPU-baseline leg."""
import json
import os
import subprocess
import sys

import pytest

import bench
import mha_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "single MI355X" in res.stderr
    assert res.stdout.strip() == ""


def test_kernel_source_hash_covers_the_kernel_sources():
    h = bench.kernel_source_sha256()
    assert len(h) == 64 and int(h, 16) >= 0
    assert bench.KERNEL_SOURCES[0] == "mha_fwd_kernel.hip"
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "head_attention_fa2_amd", "csrc", f)), f


def test_recorded_traffic_only_for_the_current_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), encoding="utf-8") as fh:
        records = json.load(fh)
    name, entry = next(iter(records.items()))
    assert entry["traffic_bytes"] > 0
    # the record applies only while the kernel sources hash to the recorded value
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: entry["kernel_source_sha256"])
    assert bench.recorded_traffic(name) == entry["traffic_bytes"]
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.recorded_traffic(name) is None
    assert bench.recorded_traffic("no_such_workload") is None


def test_recorded_traffic_is_the_scaled_counter_sum():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), encoding="utf-8") as fh:
        for entry in json.load(fh).values():
            kib = entry["fetch_kib_per_dispatch"] * entry["fetch_factor"] + \
                entry["write_kib_per_dispatch"] * entry["write_factor"]
            assert abs(kib * 1024 - entry["traffic_bytes"]) <= 1024
            # the factors are what a plain copy of known size reads and writes
            copy_kib = entry["copy_calibration_bytes"] / 1024
            assert abs(entry["fetch_factor"] * entry["copy_fetch_kib"] - copy_kib) <= 1
            assert abs(entry["write_factor"] * entry["copy_write_kib"] - copy_kib) <= 1


@pytest.mark.parametrize("name", ["fp32_B1_H2_N128_d64"])
def test_cpu_baseline_leg(name):
    w = mha_inputs.WORKLOADS[name]
    inputs = mha_inputs.draw_qkv(w)
    r = bench.cpu_baseline(w, inputs, seconds=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["cores"] >= 1 and r["value"] > 0
    assert f"of {w.B * w.H} heads" in r["sample"] and w.name in r["sample"]
