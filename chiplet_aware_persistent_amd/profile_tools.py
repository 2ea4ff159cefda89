"""Summaries of rocprofv3 output for this library's kernels.

    python -m chiplet_aware_persistent_amd.profile_tools trace <kernel_trace.csv> [--roles a,b,c] [--skip N]
    python -m chiplet_aware_persistent_amd.profile_tools traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> [--roles a,b,c] [--skip N]
    python -m chiplet_aware_persistent_amd.profile_tools sweep <config_sweep stdout> <kernel_trace.csv>
    python -m chiplet_aware_persistent_amd.profile_tools tcc <config_sweep stdout> <counter_collection.csv>
    python -m chiplet_aware_persistent_amd.profile_tools counters <config_sweep stdout> <counter_collection.csv>
    python -m chiplet_aware_persistent_amd.profile_tools read <read_probe stdout> <kernel_trace.csv>

``trace``: per-role kernel durations.  The decode projections launch the same
kernel template for several shapes, so durations are split by launch order:
with ``--bench STEPS,WARMUP`` the dispatch order of ``bench.py --steps STEPS
--warmup WARMUP`` (warm-up and timed steps launch the roles in turn, then each
role runs STEPS times back to back for its solo timing) and only the timed
steps are summarised; without it role i is every len(roles)-th dispatch and
``--skip`` drops warm-up steps.

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
    return "sg::k_gemm" in name or "sg::k_chain" in name or "sg::k_decoder" in name


def role_sequence(n: int, roles, skip: int = 0, bench=None):
    """Role of each of n dispatches (None: not summarised)."""
    if bench is None:
        return [roles[i % len(roles)] if i // len(roles) >= skip else None for i in range(n)]
    steps, warmup = bench
    seq = [roles[i % len(roles)] if i // len(roles) >= warmup else None
           for i in range((warmup + steps) * len(roles))]
    for r in roles:  # then the bench's back-to-back timing block of each role
        seq += [r + "_solo"] * steps
    assert len(seq) == n, (len(seq), n)
    return seq


def kernel_durations(trace_csv: str, roles, skip: int = 0, bench=None):
    rows = [r for r in csv.DictReader(open(trace_csv)) if _ours(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))  # the CSV is not in launch order
    per = collections.OrderedDict((r, []) for r in roles)
    if bench is not None:
        per.update((r + "_solo", []) for r in roles)
    names = {}
    for r, role in zip(rows, role_sequence(len(rows), roles, skip, bench)):
        if role is None:
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


def traffic(fetch_csv: str, write_csv: str, roles, skip: int = 0, bench=None):
    f, w = _per_dispatch(fetch_csv), _per_dispatch(write_csv)
    copies_f = [d for d in f if "copyBuffer" in d["name"]]
    copies_w = [d for d in w if "copyBuffer" in d["name"]]
    ci = max(range(len(copies_w)), key=lambda i: copies_w[i]["value"])
    true_kib = copies_w[ci]["value"]                 # bytes written == bytes read for a copy
    f_scale = true_kib / copies_f[ci]["value"]
    w_scale = 1.0
    ours_f = [d["value"] for d in f if _ours(d["name"])]
    ours_w = [d["value"] for d in w if _ours(d["name"])]
    seq_f = role_sequence(len(ours_f), roles, skip, bench)
    seq_w = role_sequence(len(ours_w), roles, skip, bench)
    out = {"calibration": {"copy_KiB": true_kib, "fetch_scale": round(f_scale, 5), "write_scale": w_scale}}
    for role in roles:
        fs = [v for v, r in zip(ours_f, seq_f) if r == role]
        ws = [v for v, r in zip(ours_w, seq_w) if r == role]
        if not fs:
            continue
        fb = statistics.mean(fs) * f_scale * 1024
        wb = statistics.mean(ws) * w_scale * 1024
        out[role] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                     "launches": len(fs)}
    return out


def _sweep_groups(sweep_log: str, rows):
    """Split dispatches of a config_sweep run into its shapes (warm-up
    launches first, then the timed ones, one JSON line per shape)."""
    shapes = [json.loads(l) for l in open(sweep_log) if l.startswith("{")]
    per = len(rows) // max(len(shapes), 1)
    assert per * len(shapes) == len(rows), (len(rows), len(shapes))
    return shapes, per


def sweep_durations(sweep_log: str, trace_csv: str, warmup: int = 6):
    rows = [r for r in csv.DictReader(open(trace_csv)) if _ours(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    shapes, per = _sweep_groups(sweep_log, rows)
    out = []
    for i, sh in enumerate(shapes):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[i * per + warmup:(i + 1) * per]]
        us = statistics.mean(d)
        wb = 2 * sh["K"] * sh["N"]
        ds = sorted(d)
        out.append({"M": sh["M"], "K": sh["K"], "N": sh["N"], "kernel": rows[i * per]["Kernel_Name"].split("(")[0],
                    "launches": len(d), "avg_us": round(us, 3), "median_us": round(statistics.median(d), 3),
                    "p10_us": round(ds[len(ds) // 10], 3), "p90_us": round(ds[min(len(ds) - 1, 9 * len(ds) // 10)], 3),
                    "weight_GBps": round(wb / us / 1e3, 1), "frac_8TBps": round(wb / us / 8e6, 4),
                    "plan": sh["plan"]})
    return out


def sweep_tcc(sweep_log: str, counter_csv: str, warmup: int = 1):
    disp = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        if not _ours(r["Kernel_Name"]):
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = [disp[k] for k in sorted(disp)]
    shapes, per = _sweep_groups(sweep_log, rows)
    out = []
    for i, sh in enumerate(shapes):
        g = rows[i * per + warmup:(i + 1) * per]
        hit = sum(x.get("TCC_HIT_sum", 0.0) for x in g)
        miss = sum(x.get("TCC_MISS_sum", 0.0) for x in g)
        r = {"M": sh["M"], "K": sh["K"], "N": sh["N"], "plan": sh["plan"]}
        if hit + miss > 0:
            r["tcc_hit"] = round(hit / (hit + miss), 4)
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in g[0]:
            # matrix-core busy cycles summed over the 1024 SIMDs, per launch; divided by
            # (kernel time x 2.4 GHz x 1024) this is the MFMA utilisation
            r["mfma_busy_cycles"] = round(sum(x["SQ_VALU_MFMA_BUSY_CYCLES"] for x in g) / len(g))
        out.append(r)
    return out


def sweep_counters(sweep_log: str, counter_csv: str, warmup: int = 1):
    """Every counter of a --pmc run of config_sweep, summed over the
    dispatch's instances and averaged over the shape's timed launches."""
    disp = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        if not _ours(r["Kernel_Name"]):
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = [disp[k] for k in sorted(disp)]
    shapes, per = _sweep_groups(sweep_log, rows)
    out = []
    for i, sh in enumerate(shapes):
        g = rows[i * per + warmup:(i + 1) * per]
        r = {"M": sh["M"], "K": sh["K"], "N": sh["N"], "plan": sh["plan"], "launches": len(g)}
        for name in sorted(g[0]) if g else []:
            r[name] = round(statistics.mean(x[name] for x in g), 1)
        out.append(r)
    return out


def read_durations(probe_log: str, trace_csv: str, warmup: int = 3):
    """Kernel durations of the read probe (k_stream_read) per (bytes, pattern)
    line of the read_probe driver's output, warm-up launches dropped."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if "k_stream_read" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    ents = [json.loads(l) for l in open(probe_log) if l.startswith("{")]
    out, pos = [], 0
    for e in ents:
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[pos + warmup:pos + e["launches"]]]
        pos += e["launches"]
        us = statistics.mean(d)
        out.append({"bytes": e["bytes"], "pattern": e["pattern"], "launches": len(d), "avg_us": round(us, 3),
                    "median_us": round(statistics.median(d), 3), "GBps": round(e["bytes"] / us / 1e3, 1),
                    "frac_8TBps": round(e["bytes"] / us / 8e6, 4)})
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--roles", default="qkv,o,gate_up,down")
    t.add_argument("--skip", type=int, default=0)
    t.add_argument("--bench", default="", help="STEPS,WARMUP of the bench.py run that was traced")
    c = sub.add_parser("traffic")
    c.add_argument("fetch")
    c.add_argument("write")
    c.add_argument("--roles", default="qkv,o,gate_up,down")
    c.add_argument("--skip", type=int, default=0)
    c.add_argument("--bench", default="", help="STEPS,WARMUP of the bench.py run that was counted")
    w = sub.add_parser("sweep")
    w.add_argument("log")
    w.add_argument("csv")
    w.add_argument("--warmup", type=int, default=6)
    h = sub.add_parser("tcc")
    h.add_argument("log")
    h.add_argument("csv")
    h.add_argument("--warmup", type=int, default=1)
    k = sub.add_parser("counters")
    k.add_argument("log")
    k.add_argument("csv")
    k.add_argument("--warmup", type=int, default=1)
    q = sub.add_parser("read")
    q.add_argument("log")
    q.add_argument("csv")
    q.add_argument("--warmup", type=int, default=3)
    a = ap.parse_args()
    if a.cmd == "read":
        print(json.dumps(read_durations(a.log, a.csv, a.warmup), indent=1))
    elif a.cmd == "sweep":
        print(json.dumps(sweep_durations(a.log, a.csv, a.warmup), indent=1))
    elif a.cmd == "counters":
        print(json.dumps(sweep_counters(a.log, a.csv, a.warmup), indent=1))
    elif a.cmd == "tcc":
        print(json.dumps(sweep_tcc(a.log, a.csv, a.warmup), indent=1))
    elif a.cmd == "trace":
        bench = tuple(int(v) for v in a.bench.split(",")) if a.bench else None
        print(json.dumps(kernel_durations(a.csv, a.roles.split(","), a.skip, bench), indent=1))
    else:
        bench = tuple(int(v) for v in a.bench.split(",")) if a.bench else None
        print(json.dumps(traffic(a.fetch, a.write, a.roles.split(","), a.skip, bench), indent=1))


if __name__ == "__main__":
    main()
