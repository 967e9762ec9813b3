"""bench.py's command line on the CPU: a multi-GPU request is refused with a
message before anything touches a GPU, and the committed counter records match
the kernel sources they were taken on (so the bench line's roofline.traffic is
reported, not silently dropped)."""
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


def test_traffic_records_match_the_current_kernel_sources():
    from quantized_moe_ffn_amd.profiling import kernel_source_hash
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        data = json.load(fh)
    assert "sage_decode" in data
    for workload, rec in data.items():
        assert rec["kernel_hash"] == kernel_source_hash(workload), workload
        assert rec["bytes_per_launch"] > 0


def test_unknown_workload_has_no_traffic():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.traffic_from_profiles("no_such_workload") is None
