"""Per-shape timing of the single decode GEMM over the benchmark configurations.

    python -m chiplet_aware_persistent_amd.config_sweep [--launches 40] [--json-overrides '{"splitk": 2}']

Shapes: the four Qwen3-8B projection shapes at M in {1, 8, 16, 32, 64}, the
K = 7168 shapes at M in {1, 2, 4, 8, 16} x N in {1536, 4096, 18432}, and the
1024 x 1024 case at M = 1.  For each shape: 6 warm-up launches, then
``--launches`` launches timed one by one with HIP events, rotating over
weight copies spanning >= 4 GiB so every launch reads its weights from HBM
(``--warm``: one buffer, so later launches find their weights in the caches).
One JSON line per shape.  Run under ``rocprofv3 --kernel-trace`` for kernel
durations without the dispatch latency the events include.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def shapes():
    out = []
    for (K, N) in [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)]:
        for M in [1, 8, 16, 32, 64]:
            out.append((M, K, N))
    for N in [1536, 4096, 18432]:
        for M in [1, 2, 4, 8, 16]:
            out.append((M, 7168, N))
    out.append((1, 1024, 1024))
    return out


def main():
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    ap = argparse.ArgumentParser()
    ap.add_argument("--launches", type=int, default=40)
    ap.add_argument("--json-overrides", default="{}")
    ap.add_argument("--only", default="", help="semicolon-separated M,K,N shapes to run instead of all")
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--warm", action="store_true",
                    help="reuse one weight buffer (warm caches) instead of rotating over >= 4 GiB of copies")
    a = ap.parse_args()
    extra = json.loads(a.json_overrides)
    dev = torch.device("cuda:0")
    cache = {}
    todo = [tuple(int(v) for v in t.split(",")) for t in a.only.split(";") if t] or shapes()
    for (M, K, N) in todo:
        wb = 2 * K * N
        copies = 1 if a.warm else max(2, -(-(4 << 30) // wb))
        if (K, N) not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            base = synth.uniform_bf16_torch(7, N, K, synth.weight_scale(K), dev)
            cache[(K, N)] = [base] + [base.clone() for _ in range(copies - 1)]
        Ws = cache[(K, N)]
        X = synth.to_torch_bf16(synth.normal_bf16(3, M, K), dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        g = sg.Gemm(M, K, N, **extra)
        ws = g.new_workspace()
        for i in range(a.warmup):
            g(X, Ws[i % copies], Y, ws)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(a.launches)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            g(X, Ws[i % copies], Y, ws)
            e1.record()
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
        med = ts[len(ts) // 2]
        p10, p90 = ts[len(ts) // 10], ts[min(len(ts) - 1, (9 * len(ts)) // 10)]
        st = g.describe()["stage"]
        print(json.dumps({"M": M, "K": K, "N": N, "us": round(med, 2), "min": round(ts[0], 2),
                          "p10": round(p10, 2), "p90": round(p90, 2), "warm": a.warm, "flags": extra.get("flags", 0),
                          "GBps": round(wb / med / 1e3, 1), "rc": g.status(ws),
                          "plan": {k: st[k] for k in ("path", "tb", "waves", "wpi", "ksl", "S", "KS", "items")}}),
              flush=True)


if __name__ == "__main__":
    main()
