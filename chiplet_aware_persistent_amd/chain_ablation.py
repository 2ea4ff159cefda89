"""Ablations of the 36-layer chain's synchronisation, same weights and inputs:

- launch granularity: one persistent launch against one launch per
  projection stage (the kernel boundary as the barrier), each enqueued
  eagerly and as a replayed HIP graph;
- completion counters: one leader per XCD polling (SGEMM_F_POLL_LEADER),
  flat counters (SGEMM_F_SYNC_FLAT), device-scope split-K arrivals
  (SGEMM_F_SYNC_AGENT);
- stage path: dot2 stages (SGEMM_F_FORCE_DOT2, M < 16) and MFMA stages
  (SGEMM_F_FORCE_MFMA) whatever the planner's choice is;
- runtime: the per-XCD scheduler workgroup releasing each task to 31
  workers through their ready-task words (SGEMM_F_SCHEDULER) against the
  static schedule in which all 32 workgroups poll the global counter.

    python -m chiplet_aware_persistent_amd.chain_ablation [--m 1 16 64] [--launches 10] [--modes ...]

Weights: the benchmarked chain's (distinct seeded U(-1/sqrt(K), 1/sqrt(K))
bf16 per layer, d = q = 4096, d_ff = 12288).  Per mode: 2 warm-up calls,
then ``--launches`` timed calls with HIP events around each on the current
stream.  One JSON line per (M, mode) with the median and the 10th and 90th
percentiles in microseconds, and whether the output equals the one-launch
output bitwise.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

D_MODEL, Q_COLS, D_FF, LAYERS = 4096, 4096, 12288, 36


def main():
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, nargs="+", default=[1, 16, 64])
    ap.add_argument("--launches", type=int, default=10)
    ap.add_argument("--modes", nargs="+", default=None, help="subset of the mode names (default: all)")
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    d, q, dff = D_MODEL, Q_COLS, D_FF
    wl = []
    for l in range(LAYERS):
        wl.append([synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WQ), q, d, synth.weight_scale(d), dev),
                   synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WO), d, q, synth.weight_scale(q), dev),
                   synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WGU), 2 * dff, d, synth.weight_scale(d), dev),
                   synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WDOWN), d, dff, synth.weight_scale(dff), dev)])
    cols = [[w[i] for w in wl] for i in range(4)]
    modes = [("one_launch", 0, False), ("launch_per_stage", sg.F_LAUNCH_PER_STAGE, False),
             ("one_launch_graph", 0, True), ("launch_per_stage_graph", sg.F_LAUNCH_PER_STAGE, True),
             ("poll_leader", sg.F_POLL_LEADER, False), ("sync_flat", sg.F_SYNC_FLAT, False),
             ("sync_agent", sg.F_SYNC_AGENT, False), ("path_dot2", sg.F_FORCE_DOT2, False),
             ("path_mfma", sg.F_FORCE_MFMA, False), ("scheduler", sg.F_SCHEDULER, False)]
    if a.modes:
        unknown = set(a.modes) - {m[0] for m in modes}
        if unknown:
            raise SystemExit("unknown modes: %s" % sorted(unknown))
        # the first mode is the reference the others are compared with bitwise
        modes = [m for m in modes if m[0] == "one_launch" or m[0] in a.modes]
    for M in a.m:
        X0 = synth.to_torch_bf16(synth.normal_bf16(synth.seed_for(5, 0, synth.T_X), M, d), dev)
        ref = None
        for name, flags, graph in modes:
            if name == "path_dot2" and M >= 16:
                continue  # no dot2 chain from M = 16 on
            ch = sg.LayerChain(M, LAYERS, d, q, dff, flags=flags)
            ws = ch.new_workspace()
            Y = torch.empty((M, d), dtype=torch.float32, device=dev)

            def call():
                ch(X0, *cols, Y, ws)

            fn = call
            if graph:
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    call()
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    call()
                fn = g.replay
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(a.launches):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            rc = ch.status(ws)
            if rc != sg.OK:
                raise RuntimeError("chain status %s (M=%d, %s)" % (sg.status_string(rc), M, name))
            if ref is None:
                ref = Y.clone()
            ts.sort()
            n = len(ts)
            print(json.dumps({"M": M, "mode": name, "path": ch.describe()["stages"][0]["path"],
                              "launches": a.launches, "median_us": round(ts[n // 2], 1),
                              "p10_us": round(ts[n // 10], 1), "p90_us": round(ts[(9 * n) // 10], 1),
                              "bitwise_equal_to_one_launch": bool(torch.equal(ref, Y))}), flush=True)


if __name__ == "__main__":
    main()
