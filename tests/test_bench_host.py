"""Host-side pieces of bench.py: the roofline record, the committed-counter lookup and the plan-derived read count.

No GPU: these run on the CPU against the library's planner and the files under profiles/.
"""
import json
import os

import pytest

import bench
import online_softmax_02_amd as osx
import synth


def test_roofline_record():
    r = bench.roofline("hbm", 6000.0, bench.PEAK_HBM_GBS, "GB/s", 123)
    assert r == {"bound": "hbm", "achieved": 6000.0, "peak": 8000.0, "unit": "GB/s", "frac": 0.75, "traffic": 123}


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_traffic_comes_from_counters_of_the_current_source(kernel):
    """traffic_for returns the committed counter bytes only while the kernel source is the one they were taken on."""
    path = os.path.join(bench.ROOT, "profiles", f"pmc_{kernel}.json")
    if not os.path.exists(path):
        assert bench.traffic_for(kernel) is None
        return
    with open(path) as f:
        rec = json.load(f)
    want = rec["traffic_bytes_per_launch"] if rec["source_sha256"] == bench.sha_of(bench.KERNEL_SOURCES[kernel]) else None
    assert bench.traffic_for(kernel) == want
    if want is not None:
        # the counted bytes are at least the algorithmic bytes (no kernel reads less than its inputs)
        assert want >= 0.99 * rec["algorithmic_bytes_per_launch"]


def test_softmax_read_count_follows_the_plan():
    """x is read twice when the planner splits the row, once when a row stays in registers."""
    assert bench.softmax_reads(osx, synth.WORKLOADS["softmax_1x16m"]) == 2
    assert bench.softmax_reads(osx, synth.WORKLOADS["softmax_causal_bf16"]) == 1
    assert bench.softmax_reads(osx, synth.WORKLOADS["softmax_4x200"]) == 1


def test_timing_statistics():
    """Per-call min / median / max come from the event windows; the mean is over all calls."""
    tm = bench.Timing(1.0, 0.25, [0.3, 0.2, 0.25, 0.22, 0.28])
    assert tm.per_call_us() == {"mean": 250.0, "min": 200.0, "median": 250.0, "max": 300.0, "windows": 5}
    assert bench.Timing(1.0, 0.5, [0.4, 0.6]).per_call_us()["median"] == 500.0
    wall, ms = tm
    assert (wall, ms) == (1.0, 0.25)


ALGORITHMIC = {  # the byte counts the bench lines divide by, from the workload definitions
    "prefill_bf16_kernel": synth.WORKLOADS["gqa_prefill_bf16"].bytes(),
    "decode_bf16_kernel": synth.WORKLOADS["gqa_decode_bf16"].bytes(),
    "softmax_split": synth.WORKLOADS["softmax_1x16m"].bytes(2),
    "softmax_wave_causal": synth.WORKLOADS["softmax_causal_bf16"].bytes(1),
    "prefill_f32_kernel": synth.WORKLOADS["attn_f32_4k_d128"].bytes(),
}


@pytest.mark.parametrize("kernel", sorted(ALGORITHMIC))
def test_profile_records_use_the_workload_byte_counts(kernel):
    """Every committed counter record states the algorithmic bytes of its workload (Q, K, V read once and O written
    once for attention; x read as often as the plan needs and y written once for the softmax)."""
    path = os.path.join(bench.ROOT, "profiles", f"pmc_{kernel}.json")
    if not os.path.exists(path):
        pytest.skip("no counter record")
    with open(path) as f:
        rec = json.load(f)
    assert rec["algorithmic_bytes_per_launch"] == int(ALGORITHMIC[kernel])


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    """One GPU only: --gpus N > 1 exits with status 2 and says so, before importing torch or touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""
