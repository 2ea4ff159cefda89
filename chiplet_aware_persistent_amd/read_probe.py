"""Attainable HBM read bandwidth on this machine: the streaming read probe
(sgemm_read_probe) over the byte counts of the decode GEMMs' weights.

    python -m chiplet_aware_persistent_amd.read_probe [--launches 20] [--warmup 3]

For each size and read order (0 grid-stride, 1 the decode GEMM's per-XCD
order): ``--warmup`` untimed and ``--launches`` timed launches, rotating over
copies spanning >= 4 GiB so every launch reads from HBM.  One JSON line per
(size, pattern) with the HIP-event median per launch; run under
``rocprofv3 --kernel-trace`` for kernel durations (summarised by
``python -m chiplet_aware_persistent_amd.profile_tools read``).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Weight bytes of the decode projections (K x N x 2): O, QKV, down, gate_up,
# and K = 7168 with N = 1536, 4096, 18432.
SIZES = [4096 * 4096 * 2, 4096 * 6144 * 2, 12288 * 4096 * 2, 4096 * 24576 * 2,
         7168 * 1536 * 2, 7168 * 4096 * 2, 7168 * 18432 * 2]


def main():
    import torch

    import chiplet_aware_persistent_amd as sg

    ap = argparse.ArgumentParser()
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    pool = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for nbytes in SIZES:
        copies = max(2, (4 << 30) // nbytes)
        bufs = [pool[i * nbytes:(i + 1) * nbytes] for i in range(copies)]
        for pattern in (0, 1):
            for i in range(a.warmup):
                sg.read_probe(bufs[i % copies], pattern, sink)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(a.launches)]
            for i, (e0, e1) in enumerate(ev):
                e0.record()
                sg.read_probe(bufs[(a.warmup + i) % copies], pattern, sink)
                e1.record()
            torch.cuda.synchronize()
            ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
            med = ts[len(ts) // 2]
            print(json.dumps({"bytes": nbytes, "pattern": pattern, "launches": a.warmup + a.launches,
                              "event_median_us": round(med, 2), "event_GBps": round(nbytes / med / 1e3, 1)}),
                  flush=True)


if __name__ == "__main__":
    main()
