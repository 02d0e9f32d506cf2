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
