"""The committed rocprofv3 summaries under profiles/ describe the current kernels.

bench.py fills `roofline.traffic` from profiles/<kernel>_<shape>_counters.txt only
when the summary was taken on the current kernel sources (it records a hash of
them). These CPU tests fail when a kernel source changes and its summaries are
not retaken, and check that every summary names the command that produced it.
"""
import os

import pytest

import bench

WORKLOADS = sorted(bench.WORKLOADS)


@pytest.mark.parametrize("workload", WORKLOADS)
def test_counter_summary_matches_current_sources(workload):
    path = bench.counters_path(workload)
    assert os.path.exists(path), f"missing {path}"
    assert bench.read_counters(workload) is not None, (
        f"{os.path.basename(path)} was taken on other kernel sources: retake the "
        f"FETCH_SIZE / WRITE_SIZE runs of --workload {workload}")


@pytest.mark.parametrize("workload", WORKLOADS)
def test_trace_summary_present_with_command(workload):
    path = os.path.join(bench.ROOT, "profiles", bench.WORKLOADS[workload]["base"] + "_kernel_trace.md")
    with open(path) as f:
        text = f.read()
    assert f"bench.py --workload {workload} " in text, "the summary must name the command that made it"
    dominant = bench.WORKLOADS[workload]["kernels"][bench.WORKLOADS[workload]["dominant"]][1]
    assert f"| {dominant} |" in text, f"no trace row for the dominant kernel {dominant}"


def test_instruction_counter_summary_covers_its_workloads():
    with open(bench.SQ_PROFILE) as f:
        rows = [line.split("|")[1].strip() for line in f if line.startswith("| ") and not line.startswith("| workload")]
    assert sorted(r for r in rows if r in bench.SQ_ELEMENTS) == sorted(bench.SQ_ELEMENTS)
    for w in bench.SQ_ELEMENTS:
        assert bench.valu_ops_per_element(w) is not None
