"""Host logic of quantized_moe_ffn_amd.profiling on small hand-made rocprofv3 CSVs.

The module turns rocprofv3 output into the profile summaries and the HBM
traffic records that bench.py reports; these tests check its arithmetic on
inputs whose answers are worked out by hand: kernel-name shortening, the
ns -> us statistics, the layer-call period over steps, per-dispatch counter
means, the copy calibration and the traffic record it writes.  CPU only.
"""
import csv
import json
import os

import pytest

from quantized_moe_ffn_amd import profiling as pf


def _write(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_short_name_drops_namespaces_and_arguments():
    assert pf.short_name("void moe::(anonymous namespace)::gateup_mfma_kernel<2, 12>(moe::MfmaArgs)") == \
        "gateup_mfma_kernel<2, 12>"
    assert pf.short_name("void moe::dec_down_kernel<12, 16, 2>(moe::DecArgs)") == "dec_down_kernel<12, 16, 2>"


def test_kernel_stats_filters_and_converts_to_microseconds(tmp_path):
    _write(tmp_path / "kt_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"], [
        ["void moe::dec_down_kernel<12, 16, 2>(moe::DecArgs)", 40, 5250.0, 4200.0, 8100.0],
        ["void at::native::elementwise_kernel<128, 4>(int)", 7, 1000.0, 900.0, 1100.0],
    ])
    got = pf.kernel_stats(str(tmp_path), "dec_")
    assert got == [("dec_down_kernel<12, 16, 2>", 40, 5.25, 4.2, 8.1)]


def test_layer_period_is_the_median_over_steps(tmp_path):
    # two layer calls per step; step s spans first-kernel start to last-kernel end
    rows = []
    starts = [0, 30000, 100000, 128000, 200000, 236000]   # three steps
    for i, t0 in enumerate(starts):
        rows.append(["void moe::dec_gateup_pipe_kernel<8>(moe::DecArgs, int)", t0, t0 + 7000])
        rows.append(["void moe::dec_down_kernel<12>(moe::DecArgs)", t0 + 8000, t0 + 13000])
    rows.reverse()   # the module sorts by start time
    _write(tmp_path / "kt_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    per, n = pf.layer_period_us(str(tmp_path), "dec_gateup", "dec_down", 2)
    # steps: (30000+13000-0)/2 = 21.5 us, (128000+13000-100000)/2 = 20.5 us, (236000+13000-200000)/2 = 24.5 us
    assert n == 3 and per == pytest.approx(21.5)


def _counters(path, counter, rows):
    _write(path, ["Kernel_Name", "Counter_Name", "Counter_Value"],
           [[k, counter, v] for k, v in rows])


def test_counter_means_and_copy_scale(tmp_path):
    _counters(tmp_path / "c_counter_collection.csv", "FETCH_SIZE", [
        ["void moe::k1(moe::DecArgs)", 100.0], ["void moe::k1(moe::DecArgs)", 300.0],
        ["void moe::k2(moe::DecArgs)", 50.0],
    ])
    means = pf.counter_means(str(tmp_path), "FETCH_SIZE", "moe::")
    assert means == {"k1": (200.0, 2), "k2": (50.0, 1)}
    cal = tmp_path / "cal"
    cal.mkdir()
    _counters(cal / "f_counter_collection.csv", "FETCH_SIZE", [["__amd_rocclr_copyBuffer", 524288.0]])
    assert pf.copy_scale(str(cal), "FETCH_SIZE", 1 << 30) == pytest.approx(2048.0)
    _counters(cal / "f_counter_collection.csv", "FETCH_SIZE", [])
    with pytest.raises(ValueError):
        pf.copy_scale(str(cal), "FETCH_SIZE", 1 << 30)


def test_traffic_record(tmp_path):
    d = {n: tmp_path / n for n in ("fetch", "write", "cal_fetch", "cal_write")}
    for p in d.values():
        p.mkdir()
    _counters(d["fetch"] / "f_counter_collection.csv", "FETCH_SIZE", [
        ["void moe::dec_gateup_pipe_kernel<8>(moe::DecArgs, int)", 4000.0],
        ["void moe::dec_gateup_pipe_kernel<8>(moe::DecArgs, int)", 6000.0],
        ["void moe::dec_down_kernel<12>(moe::DecArgs)", 2500.0],
    ])
    _counters(d["write"] / "w_counter_collection.csv", "WRITE_SIZE", [
        ["void moe::dec_down_kernel<12>(moe::DecArgs)", 10.0],
    ])
    # copies of 1 GiB: 2^20 FETCH units -> 1024 B per unit; 2^19 WRITE units -> 2048 B per unit
    _counters(d["cal_fetch"] / "f_counter_collection.csv", "FETCH_SIZE", [["__amd_rocclr_copyBuffer", 1 << 20]])
    _counters(d["cal_write"] / "w_counter_collection.csv", "WRITE_SIZE", [["__amd_rocclr_copyBuffer", 1 << 19]])
    out = tmp_path / "traffic.json"
    rc = pf.main(["traffic", "--workload", "sage_decode", "--fetch", str(d["fetch"]), "--write", str(d["write"]),
                  "--cal-fetch", str(d["cal_fetch"]), "--cal-write", str(d["cal_write"]), "--out", str(out)])
    assert rc == 0
    rec = json.load(open(out))["sage_decode"]
    assert rec["fetch_scale_bytes_per_unit"] == 1024.0 and rec["write_scale_bytes_per_unit"] == 2048.0
    k1 = rec["kernels"]["dec_gateup_pipe_kernel<8>"]
    k2 = rec["kernels"]["dec_down_kernel<12>"]
    assert (k1["fetch_bytes"], k1["write_bytes"], k1["dispatches"]) == (5000 * 1024, 0, 2)
    assert (k2["fetch_bytes"], k2["write_bytes"], k2["dispatches"]) == (2500 * 1024, 10 * 2048, 1)
    assert rec["bytes_per_launch"] == 7500 * 1024 + 10 * 2048
    assert rec["kernel_hash"] == pf.kernel_source_hash("sage_decode")
    assert rec["kernel_files"] == pf.kernel_files("sage_decode")
    # a second workload is added beside the first, not over it
    rc = pf.main(["traffic", "--workload", "mtp_window", "--fetch", str(d["fetch"]), "--write", str(d["write"]),
                  "--cal-fetch", str(d["cal_fetch"]), "--cal-write", str(d["cal_write"]), "--out", str(out)])
    assert rc == 0 and set(json.load(open(out))) == {"sage_decode", "mtp_window"}
