"""Reduces rocprofv3 CSV output to the figures the benchmark reports.

Two uses:
  * ``stats``: the per-kernel rows of a ``--kernel-trace --stats`` run
    (``*_kernel_stats.csv``) as a short text table, with the layer-call period
    derived from the kernel trace (``*_kernel_trace.csv``).
  * ``traffic``: HBM bytes per layer call from two ``--pmc`` runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch) over the library's kernels, each scaled
    by what the same counter reads for a device-to-device copy of known size.
    The record goes into ``profiles/traffic.json`` keyed by the workload name and
    tagged with a hash of the sources of that workload's kernels, so a reader
    can tell when they have changed since the counters were taken.

Only reads CSV files; runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


# Sources of each path's kernels (plus the API layer that launches them).
_COMMON = ("common.h", "kernels.h", "libmoe.hip", "moe_api.hip", "route.hip")
_DECODE = _COMMON + ("qblock.h", "decode_fused.hip")
_INT8 = _COMMON + ("quant.hip", "ffn_mfma.hip", "ffn_int8.hip", "ffn_decode.hip")


# A workload run with MOE_FFN_PAIR_BF16 is recorded under its name with this suffix.
PAIR_BF16_SUFFIX = "+pair_bf16"


def kernel_files(workload: str | None = None):
    """The library sources a workload's kernels are built from (all sources when None)."""
    if workload is None:
        return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    from quantized_moe_ffn_amd import synth
    if workload.endswith(PAIR_BF16_SUFFIX):
        workload = workload[:-len(PAIR_BF16_SUFFIX)]
    return sorted(_INT8 if synth.WORKLOADS[workload].int8_path else _DECODE)


def kernel_source_hash(workload: str | None = None) -> str:
    """Hash of the named sources (names and bytes) of a workload's kernel path."""
    h = hashlib.sha256()
    for f in kernel_files(workload):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _rows(path: str):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def short_name(name: str) -> str:
    """Kernel name without the argument list and namespace."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
    return base.replace("moe::", "")


def kernel_stats(run_dir: str, name_re: str):
    """(short name, calls, average us, min us, max us) of the matching kernels."""
    out = []
    for r in _rows(_one(os.path.join(run_dir, "*kernel_stats.csv"))):
        if re.search(name_re, r["Name"]):
            out.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                        float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return out


def layer_period_us(run_dir: str, first_re: str, last_re: str, per_step: int):
    """Median over steps of (last kernel end - first kernel start) / calls, where
    a step is ``per_step`` consecutive pairs of first/last kernels in the trace.
    Returns (median period, number of steps seen)."""
    rows = _rows(_one(os.path.join(run_dir, "*kernel_trace.csv")))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    firsts = [r for r in rows if re.search(first_re, r["Kernel_Name"])]
    lasts = [r for r in rows if re.search(last_re, r["Kernel_Name"])]
    n = min(len(firsts), len(lasts)) // per_step
    periods = []
    for s in range(n):
        a = int(firsts[s * per_step]["Start_Timestamp"])
        b = int(lasts[s * per_step + per_step - 1]["End_Timestamp"])
        periods.append((b - a) / 1e3 / per_step)
    return (statistics.median(periods) if periods else None), n


def counter_means(run_dir: str, counter: str, name_re: str):
    """Mean counter value per dispatch for every matching kernel name."""
    acc = {}
    for r in _rows(_one(os.path.join(run_dir, "*counter_collection.csv"))):
        if r["Counter_Name"] != counter or not re.search(name_re, r["Kernel_Name"]):
            continue
        acc.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (statistics.fmean(v), len(v)) for k, v in acc.items()}


def copy_scale(run_dir: str, counter: str, copy_bytes: int, name_re: str = "copyBuffer") -> float:
    """Bytes per counter unit, from a copy of copy_bytes bytes (reads and writes copy_bytes)."""
    vals = counter_means(run_dir, counter, name_re)
    if len(vals) != 1:
        raise ValueError("expected one copy kernel in %s, found %s" % (run_dir, list(vals)))
    (mean, _), = vals.values()
    return copy_bytes / mean


def cmd_stats(a) -> int:
    print("kernel | calls | avg us | min us | max us")
    for name, calls, avg, mn, mx in kernel_stats(a.run, a.kernels):
        print("%s | %d | %.3f | %.3f | %.3f" % (name, calls, avg, mn, mx))
    if a.first and a.last:
        per, n = layer_period_us(a.run, a.first, a.last, a.per_step)
        if per is not None:
            print("layer-call period from the trace (median over %d steps of %d calls): %.3f us"
                  % (n, a.per_step, per))
    return 0


def cmd_traffic(a) -> int:
    fs = copy_scale(a.cal_fetch, "FETCH_SIZE", a.copy_bytes)
    ws = copy_scale(a.cal_write, "WRITE_SIZE", a.copy_bytes)
    fetch = counter_means(a.fetch, "FETCH_SIZE", a.kernels)
    write = counter_means(a.write, "WRITE_SIZE", a.kernels)
    kernels = {}
    total = 0.0
    for name in sorted(set(fetch) | set(write)):
        f = fetch.get(name, (0.0, 0))[0] * fs
        w = write.get(name, (0.0, 0))[0] * ws
        kernels[name] = {"fetch_bytes": round(f), "write_bytes": round(w),
                         "dispatches": max(fetch.get(name, (0, 0))[1], write.get(name, (0, 0))[1])}
        total += f + w
    rec = {"kernel_hash": kernel_source_hash(a.workload), "kernel_files": kernel_files(a.workload),
           "bytes_per_launch": round(total),
           "fetch_scale_bytes_per_unit": round(fs, 3), "write_scale_bytes_per_unit": round(ws, 3),
           "copy_bytes": a.copy_bytes, "kernels": kernels}
    data = {}
    if os.path.exists(a.out):
        with open(a.out) as fh:
            data = json.load(fh)
    data[a.workload] = rec
    with open(a.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    json.dump({a.workload: rec}, sys.stdout, indent=1)
    print()
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats", help="kernel-trace statistics as text")
    s.add_argument("run", help="rocprofv3 output directory of a --kernel-trace --stats run")
    s.add_argument("--kernels", default=r"moe::", help="regex over kernel names")
    s.add_argument("--first", help="regex of the first kernel of a layer call")
    s.add_argument("--last", help="regex of the last kernel of a layer call")
    s.add_argument("--per-step", type=int, default=40, help="layer calls per step")
    t = sub.add_parser("traffic", help="HBM bytes per layer call from FETCH_SIZE/WRITE_SIZE runs")
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True, help="rocprofv3 directory of the FETCH_SIZE run")
    t.add_argument("--write", required=True, help="rocprofv3 directory of the WRITE_SIZE run")
    t.add_argument("--cal-fetch", required=True, help="FETCH_SIZE run over the calibration copy")
    t.add_argument("--cal-write", required=True, help="WRITE_SIZE run over the calibration copy")
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--kernels", default=r"moe::")
    t.add_argument("--out", default=os.path.join(os.path.dirname(HERE), "profiles", "traffic.json"))
    a = ap.parse_args(argv)
    return cmd_stats(a) if a.cmd == "stats" else cmd_traffic(a)


if __name__ == "__main__":
    sys.exit(main())
