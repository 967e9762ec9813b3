"""bench.py's command line on the CPU: a multi-GPU request is refused with a
message before anything touches a GPU, and a committed counter record is
reported only while the kernel sources it was taken on are unchanged."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_kernel_sources_it_was_taken_on():
    """A counter record carries the hash of its workload's kernel sources; bench.py reports
    its bytes while that hash matches the sources and null once they have changed."""
    sys.path.insert(0, ROOT)
    import bench
    from quantized_moe_ffn_amd.profiling import kernel_source_hash
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        data = json.load(fh)
    assert data
    for workload, rec in data.items():
        assert rec["bytes_per_launch"] > 0 and len(rec["kernel_hash"]) == 16
        got = bench.traffic_from_profiles(workload)
        if rec["kernel_hash"] == kernel_source_hash(workload):
            assert got == rec["bytes_per_launch"], workload
        else:
            assert got is None, workload


def test_unknown_workload_has_no_traffic():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.traffic_from_profiles("no_such_workload") is None
