"""Host-side parts of bench.py that need no GPU: the one-GPU guard, the recorded-counter
lookup keyed by the kernel sources' hash, the oracle's CPU-baseline leg and the full
parity check over the heads it evaluated."""
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


COUNTERS = os.path.join(ROOT, "profiles", "kernel_counters.json")


def test_recorded_counters_only_for_the_current_sources(monkeypatch):
    with open(COUNTERS, encoding="utf-8") as fh:
        records = json.load(fh)
    name, entry = next(iter(records.items()))
    assert entry["traffic_bytes"] > 0
    # the record applies only while the kernel sources hash to the recorded value
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: entry["kernel_source_sha256"])
    got = bench.recorded_counters(name)
    assert got["traffic_bytes"] == entry["traffic_bytes"]
    assert got["mfma_busy"] == entry.get("mfma_busy")
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert set(bench.recorded_counters(name).values()) == {None}
    assert set(bench.recorded_counters("no_such_workload").values()) == {None}


def test_recorded_traffic_is_the_scaled_counter_sum():
    with open(COUNTERS, encoding="utf-8") as fh:
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
    r, heads = bench.cpu_baseline(w, inputs, seconds=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["cores"] >= 1 and r["value"] > 0
    assert f"of {w.B * w.H} heads" in r["sample"] and w.name in r["sample"]
    assert heads and all(h1 > h0 for _, h0, h1, _, _ in heads)


def test_host_workers_respects_the_cpu_share(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_workers() == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_workers() == n


def test_parity_full_compares_every_element():
    import numpy as np
    import torch

    import oracle

    w = mha_inputs.WORKLOADS["fp32_B1_H2_N128_d64"]
    q, k, v = mha_inputs.draw_qkv(w)
    _, heads = bench.cpu_baseline(w, (q, k, v), seconds=1e9)
    o_ref, l_ref = oracle.attention_forward(oracle.decode(q, "f32"), oracle.decode(k, "f32"),
                                            oracle.decode(v, "f32"), causal=w.causal, scale=w.scale)
    o, lse = torch.from_numpy(o_ref.astype(np.float32)), torch.from_numpy(l_ref.astype(np.float32))
    r = bench.parity_full(w, (o, lse), heads)
    assert r["rows"] == r["of_rows"] == w.B * w.H * w.N
    assert r["max_abs_dO"] < 1e-6 and r["max_abs_dLSE"] < 1e-5
    # a single wrong element anywhere is seen
    o[0, 1, 77, 5] += 0.5
    assert bench.parity_full(w, (o, lse), heads)["max_abs_dO"] >= 0.5 - 1e-6
