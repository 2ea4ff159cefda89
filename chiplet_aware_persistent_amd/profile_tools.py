"""Summaries of rocprofv3 output for this library's kernels.

    python -m chiplet_aware_persistent_amd.profile_tools trace <kernel_trace.csv> [--roles a,b,c] [--skip N]
    python -m chiplet_aware_persistent_amd.profile_tools traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> [--roles a,b,c] [--skip N]

``trace``: per-role kernel durations.  The decode projections launch the same
kernel template for several shapes, so durations are split by launch order
(role i = every len(roles)-th sgemm/chain dispatch); ``--skip`` drops warm-up
steps.

``traffic``: HBM bytes per launch from the FETCH_SIZE and WRITE_SIZE counters
(KiB per dispatch), each scaled by what the same counter reads for the largest
plain device copy in the run (``__amd_rocclr_copyBuffer``: its true bytes read
and written are both equal to the bytes it writes, which WRITE_SIZE reports
exactly).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import statistics


def _ours(name: str) -> bool:
    return "sg::k_gemm" in name or "sg::k_chain" in name


def kernel_durations(trace_csv: str, roles, skip: int = 0):
    rows = [r for r in csv.DictReader(open(trace_csv)) if _ours(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))  # the CSV is not in launch order
    per = collections.OrderedDict((r, []) for r in roles)
    names = {}
    for i, r in enumerate(rows):
        role = roles[i % len(roles)]
        if i // len(roles) < skip:
            continue
        per[role].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        names[role] = r["Kernel_Name"].split("(")[0]
    out = {}
    for role, v in per.items():
        if not v:
            continue
        out[role] = {"kernel": names[role], "launches": len(v), "avg_us": round(statistics.mean(v), 3),
                     "median_us": round(statistics.median(v), 3), "min_us": round(min(v), 3),
                     "max_us": round(max(v), 3)}
    return out


def _per_dispatch(counter_csv: str):
    disp = {}
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "value": 0.0})
        d["value"] += float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def traffic(fetch_csv: str, write_csv: str, roles, skip: int = 0):
    f, w = _per_dispatch(fetch_csv), _per_dispatch(write_csv)
    copies_f = [d for d in f if "copyBuffer" in d["name"]]
    copies_w = [d for d in w if "copyBuffer" in d["name"]]
    ci = max(range(len(copies_w)), key=lambda i: copies_w[i]["value"])
    true_kib = copies_w[ci]["value"]                 # bytes written == bytes read for a copy
    f_scale = true_kib / copies_f[ci]["value"]
    w_scale = 1.0
    ours_f = [d["value"] for d in f if _ours(d["name"])]
    ours_w = [d["value"] for d in w if _ours(d["name"])]
    out = {"calibration": {"copy_KiB": true_kib, "fetch_scale": round(f_scale, 5), "write_scale": w_scale}}
    for j, role in enumerate(roles):
        fs = [v for i, v in enumerate(ours_f) if i % len(roles) == j and i // len(roles) >= skip]
        ws = [v for i, v in enumerate(ours_w) if i % len(roles) == j and i // len(roles) >= skip]
        if not fs:
            continue
        fb = statistics.mean(fs) * f_scale * 1024
        wb = statistics.mean(ws) * w_scale * 1024
        out[role] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                     "launches": len(fs)}
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--roles", default="qkv,o,gate_up,down")
    t.add_argument("--skip", type=int, default=0)
    c = sub.add_parser("traffic")
    c.add_argument("fetch")
    c.add_argument("write")
    c.add_argument("--roles", default="qkv,o,gate_up,down")
    c.add_argument("--skip", type=int, default=0)
    a = ap.parse_args()
    roles = a.roles.split(",")
    if a.cmd == "trace":
        print(json.dumps(kernel_durations(a.csv, roles, a.skip), indent=1))
    else:
        print(json.dumps(traffic(a.fetch, a.write, roles, a.skip), indent=1))


if __name__ == "__main__":
    main()
