#!/usr/bin/env python3
"""Benchmark of the small-M decode GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload proj|chain] [--sweep]

Default workload ("proj"): the Qwen3-8B-shaped decode projections at M = 1
(QKV 4096x6144, O 4096x4096, gate_up 4096x24576, down 12288x4096; 368 MiB of
bf16 weights).  One step = one sgemm_run of each projection on one batch of
synthetic input.  Weights rotate over enough copies (>= 1 GiB) that no launch
finds its weights in the 256 MB Infinity Cache or the L2s: every step streams
its weights from HBM (the rotation spans >= 4 GiB: with only ~1 GiB some
launches still hit the 256 MB Infinity Cache).  ``value`` is weight bytes moved per second over the
timed steps (GB/s); ``roofline`` reports the dominant kernel (gate_up) against
the 8 TB/s HBM peak, its launch durations measured with HIP events on the
launch stream, next to the attainable rate of a plain streaming read of the
same weight buffers (sgemm_read_probe); ``cpu_baseline`` is the CPU oracle on
the same step.

Unless ``--no-extra`` is given, the line also carries ``configs``: every
other configuration timed in the same run with HIP events on the launch
stream (the single GEMM at M = 1, 8, 16, 32, 64, 128, 256 on the four
projection shapes, the K = 7168 grid at M = 1..16 and at M = 256 x 18432,
1 x 1024 x 1024, each on weights rotating over a 4.5 GiB pool; the 36-layer
chain at M = 64, 16 and 1), each with its fraction of 8 TB/s (and, for the
single GEMM, its TFLOP/s and its fraction of the roofline floor, the longer
of the weight bytes at 8 TB/s and the flops at 2.5 PFLOP/s).

``--workload chain``: the 36-layer persistent chain at M = 64 (``--chain-m``
selects another row count; Q 4096x4096,
O 4096x4096, gate_up 4096x24576 with SiLU gate, down 12288x4096 per layer;
13.29 GB of weights) in one launch per step.  ``--workload decoder``: the
whole decoder layer (RMSNorm, QKV 4096x6144, grouped-query decode attention
over a synthetic KV cache of ``--decoder-ctx`` positions with 32 query and 8
key/value heads of 128, O with residual, RMSNorm, gate_up with SiLU gate, down
with residual), 36 layers in one launch, at M = ``--chain-m`` rows.  ``--chain-kchunk`` runs every
chain stage on the K-chunked MFMA path and ``--chain-tn`` fixes the planner's
tile width (ablations of the chain's stage kernels).

Prints exactly one JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROJ = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 24576), ("down", 12288, 4096)]
HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_src_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chiplet_aware_persistent_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(name: str):
    """HBM traffic per launch from the committed rocprofv3 PMC summary, or None
    when the kernels changed since it was taken."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_src_hash") != kernel_src_hash():
        return None
    return t.get("bytes_per_launch")


def host_cpu():
    """CPU model name and the host's logical CPU count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def cpu_baseline_proj(x_bits, w_host):
    import oracle

    t0 = time.perf_counter()
    reps = 0
    wbytes = 0
    while True:
        for (name, K, N), w in zip(PROJ, w_host):
            oracle.gemm(x_bits[K], w, want_abs=False)
            wbytes += 2 * K * N
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 2000:
            break
    dt = time.perf_counter() - t0
    return dict({"value": round(wbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                 "kind": "oracle",
                 "sample": "%d full steps (%.1f s): all four projections, every output column, M=1, double "
                           "accumulation" % (reps, dt)}, **host_cpu())


def cpu_baseline_chain(M, x_bits, layer_w):
    """The oracle's chain layer (Q, O, gate_up with SiLU gate, down) on the
    host cores, repeated on layer 0's weights for about 10 s."""
    import oracle

    t0 = time.perf_counter()
    reps = 0
    wbytes = 0
    layer_bytes = sum(2 * w.size for w in layer_w)
    while True:
        oracle.layer(x_bits, *layer_w)
        wbytes += layer_bytes
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 2000:
            break
    dt = time.perf_counter() - t0
    return dict({"value": round(wbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                 "kind": "oracle",
                 "sample": "%d chain layers (%.1f s) on layer 0's weights and input: Q, O, gate_up with SiLU "
                           "gate, down, every output column, M=%d, double accumulation" % (reps, dt, M)},
                **host_cpu())


def bench_proj(args):
    import numpy as np
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    dev = torch.device("cuda:0")
    M = 1
    wbytes_step = sum(2 * K * N for _, K, N in PROJ)
    copies = max(2, -(-(4 << 30) // wbytes_step))
    log("proj: %d weight copies (%.1f MiB each set)" % (copies, wbytes_step / 2 ** 20))
    W = []  # W[copy][proj]
    for c in range(copies):
        ws_ = []
        for i, (name, K, N) in enumerate(PROJ):
            seed = synth.seed_for(2, 0, 1 + i)
            t = synth.uniform_bf16_torch(seed, N, K, synth.weight_scale(K), dev)
            ws_.append(t)
        W.append(ws_)
    x_bits = {K: synth.normal_bf16(synth.seed_for(2, 0, synth.T_X, K % 16), M, K) for _, K, _ in PROJ}
    X = {K: synth.to_torch_bf16(b, dev) for K, b in x_bits.items()}
    plans = [sg.Gemm(M, K, N) for _, K, N in PROJ]
    wss = [p.new_workspace() for p in plans]
    Y = [torch.empty((M, N), dtype=torch.float32, device=dev) for _, _, N in PROJ]
    stream = torch.cuda.current_stream()
    h = int(stream.cuda_stream)
    lib = sg.library()
    ptrs = [[(plans[i].handle, X[K].data_ptr(), W[c][i].data_ptr(), Y[i].data_ptr(), wss[i].data_ptr())
             for i, (_, K, _) in enumerate(PROJ)] for c in range(copies)]

    def step(c, events=None):
        for i, a in enumerate(ptrs[c]):
            if events is not None:
                events[i][0].record(stream)
            rc = lib.sgemm_run(*a, h)
            if rc:
                raise sg.SgemmError(rc, "sgemm_run")
            if events is not None:
                events[i][1].record(stream)

    if args.copy_calibration:
        # A plain device copy of known size, for scaling the FETCH_SIZE /
        # WRITE_SIZE counters of a --pmc run (read 256 MiB, write 256 MiB).
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for s in range(args.warmup):
        step(s % copies)
    torch.cuda.synchronize()
    # timed region: K steps, wall clock
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s % copies)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-kernel durations with HIP events on the launch stream: each
    # projection launched back to back `steps` times (rotating weight copies)
    # between two events; per-launch time = elapsed / steps.  Bracketing single
    # launches would add the dispatch latency (~2-3 us) to every figure.
    per = {}
    for i, (name, K, N) in enumerate(PROJ):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a = ptrs[0][i]
        e0.record(stream)
        for s in range(args.steps):
            rc = lib.sgemm_run(ptrs[s % copies][i][0], a[1], ptrs[s % copies][i][2], a[3], a[4], h)
            if rc:
                raise sg.SgemmError(rc, "sgemm_run")
        e1.record(stream)
        torch.cuda.synchronize()
        avg = e0.elapsed_time(e1) * 1e3 / args.steps  # us
        per[name] = {"K": K, "N": N, "us_avg": round(avg, 3),
                     "weight_GBps": round(2 * K * N / (avg * 1e-6) / 1e9, 1),
                     "plan": plans[i].describe()["stage"]}
    for i, p in enumerate(plans):
        rc = p.status(wss[i])
        if rc:
            raise sg.SgemmError(rc, "status")
    # Attainable reference for the dominant projection: the streaming read
    # probe over the same weight buffers (same rotation, launched back to
    # back), in the GEMM's per-XCD order and in grid-stride order.
    dom = max(per, key=lambda k: per[k]["us_avg"])
    di = [n for n, _, _ in PROJ].index(dom)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    attain = {}
    for pattern, key in ((1, "GBps_gemm_order"), (0, "GBps_grid_stride")):
        for s in range(args.warmup):
            sg.read_probe(W[s % copies][di], pattern, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            sg.read_probe(W[s % copies][di], pattern, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        attain[key] = round(W[0][di].numel() * 2 / (us * 1e-6) / 1e9, 1)
    w_host = [synth.from_torch_bf16(W[0][i]) for i in range(len(PROJ))] if not args.no_cpu else None
    ms_step = wall / args.steps * 1e3
    value = wbytes_step / (wall / args.steps) / 1e9
    K, N = per[dom]["K"], per[dom]["N"]
    alg = 2 * K * N + 2 * M * K + 4 * M * N
    achieved = alg / (per[dom]["us_avg"] * 1e-6) / 1e9
    traffic = load_traffic("gemm_dot2_m1_gate_up")
    out = {
        "metric": "achieved HBM GB/s (weight bytes) and us per decode GEMM, M=1-64 bf16",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_8b_decode_projections_m1", "M": M,
                   "shapes_KxN": [[K_, N_] for _, K_, N_ in PROJ], "weight_bytes_per_step": wbytes_step,
                   "cold_hbm_weight_copies": copies, "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "kernel": "sgemm dot2 %s %dx%d" % (dom, K, N),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg, "avg_launch_us": per[dom]["us_avg"],
                     "attainable": dict(attain, kernel="sgemm_read_probe over the same weight buffers"),
                     "frac_of_attainable": round(achieved / attain["GBps_gemm_order"], 4)},
        "per_gemm": {k: {kk: v for kk, v in d.items() if kk != "plan"} for k, d in per.items()},
        "plans": {k: {kk: d["plan"][kk] for kk in ("path", "waves", "TN", "ksl", "S", "KS", "items")}
                  for k, d in per.items()},
    }
    if not args.no_extra:
        # The other configurations, each timed on the same box in this run:
        # every single-GEMM shape (M = 1..64 on the decode projections, the
        # K = 7168 grid, 1 x 1024 x 1024) and the 36-layer chain at M = 64 and 1.
        del W, ptrs
        torch.cuda.empty_cache()
        out["configs"] = {"gemm": timed_gemm_table(dev, max(args.steps, 20), args.warmup)}
        wl = chain_weights(dev)
        out["configs"]["chain36"] = [timed_chain(dev, wl, m, 10, 2) for m in (64, 16, 1)]
        del wl
        torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_proj(x_bits, w_host)
    return out


GEMM_TABLE = ([(1, 1024, 1024)] +
              [(M, K, N) for M in (1, 8, 16, 32, 64, 128, 256) for _, K, N in PROJ] +
              [(M, 7168, N) for M in (1, 2, 4, 8, 16) for N in (1536, 4096, 18432)] +
              [(256, 7168, 18432)])
MFMA_BF16_PEAK_TFLOPS = 2500.0


def timed_gemm_table(dev, steps, warmup):
    """Every single-GEMM configuration shape: kernel time per launch from HIP
    events around `steps` back-to-back launches on the launch stream, the
    weights rotating over views of a >= 4 GiB pool so each launch reads them
    from HBM."""
    import torch

    import chiplet_aware_persistent_amd as sg

    pool = torch.empty((9 << 30) // 4, dtype=torch.bfloat16, device=dev)   # 4.5 GiB
    pool.uniform_(-0.01, 0.01)
    stream = torch.cuda.current_stream()
    lib, h = sg.library(), int(stream.cuda_stream)
    rows = []
    for M, K, N in GEMM_TABLE:
        g = sg.Gemm(M, K, N)
        ws = g.new_workspace()
        X = torch.randn((M, K), device=dev).to(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        span = -(-N * K // 256) * 256
        copies = min(pool.numel() // span, 4096)
        ptr = [pool.data_ptr() + c * span * 2 for c in range(copies)]
        a = (g.handle, X.data_ptr(), 0, Y.data_ptr(), ws.data_ptr(), h)
        for s_ in range(warmup):
            lib.sgemm_run(a[0], a[1], ptr[s_ % copies], a[3], a[4], h)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s_ in range(steps):
            rc = lib.sgemm_run(a[0], a[1], ptr[(warmup + s_) % copies], a[3], a[4], h)
            if rc:
                raise sg.SgemmError(rc, "sgemm_run")
        e1.record(stream)
        torch.cuda.synchronize()
        rc = g.status(ws)
        if rc:
            raise sg.SgemmError(rc, "status")
        us = e0.elapsed_time(e1) * 1e3 / steps
        st = g.describe()["stage"]
        # Roofline floor: the weight bytes at 8 TB/s or the 2 M K N flops at
        # the dense bf16 matrix-core peak, whichever is longer (the latter
        # only matters from M of about 300 up; M = 128 and 256 lean towards it).
        floor_us = max(2 * K * N / (HBM_PEAK_GBPS * 1e3), 2.0 * M * K * N / (MFMA_BF16_PEAK_TFLOPS * 1e6))
        rows.append({"M": M, "K": K, "N": N, "us_avg": round(us, 3),
                     "weight_GBps": round(2 * K * N / (us * 1e-6) / 1e9, 1),
                     "frac_of_8TBps": round(2 * K * N / (us * 1e-6) / 1e12 / 8.0, 4),
                     "tflops": round(2.0 * M * K * N / (us * 1e-6) / 1e12, 1),
                     "frac_of_roofline": round(floor_us / us, 4),
                     "plan": "%s ta=%d tb=%d wpi=%d ksl=%d S=%d" % (st["path"], st["ta"], st["tb"], st["wpi"],
                                                                   st["ksl"], st["S"])})
        log("table %dx%dx%d: %.2f us" % (M, K, N, us))
    del pool
    torch.cuda.empty_cache()
    return rows


def chain_weights(dev, L=36, d=4096, q=4096, dff=12288):
    import synth

    return [[synth.uniform_bf16_torch(synth.seed_for(5, l, 1), q, d, synth.weight_scale(d), dev),
             synth.uniform_bf16_torch(synth.seed_for(5, l, 2), d, q, synth.weight_scale(q), dev),
             synth.uniform_bf16_torch(synth.seed_for(5, l, 3), 2 * dff, d, synth.weight_scale(d), dev),
             synth.uniform_bf16_torch(synth.seed_for(5, l, 4), d, dff, synth.weight_scale(dff), dev)]
            for l in range(L)]


def timed_chain(dev, wl, M, steps, warmup):
    """The 36-layer chain at M rows: per-launch time from HIP event pairs."""
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    L, d, q, dff = len(wl), wl[0][0].shape[1], wl[0][0].shape[0], wl[0][3].shape[1]
    X0 = synth.to_torch_bf16(synth.normal_bf16(synth.seed_for(5, 0, 0), M, d), dev)
    ch = sg.LayerChain(M, L, d, q, dff)
    ws = ch.new_workspace()
    Y = torch.empty((M, d), dtype=torch.float32, device=dev)
    cols = [[w[i] for w in wl] for i in range(4)]
    for _ in range(warmup):
        ch(X0, *cols, Y, ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s_ in range(steps):
        ev[s_][0].record()
        ch(X0, *cols, Y, ws)
        ev[s_][1].record()
    torch.cuda.synchronize()
    rc = ch.status(ws)
    if rc:
        raise sg.SgemmError(rc, "chain status")
    ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    wbytes = L * 2 * (q * d + d * q + 2 * dff * d + d * dff)
    avg = sum(ts) / len(ts)
    return {"M": M, "layers": L, "us_avg": round(avg, 2), "us_median": round(ts[len(ts) // 2], 2),
            "weight_GBps": round(wbytes / (avg * 1e-6) / 1e9, 1),
            "frac_of_8TBps": round(wbytes / (avg * 1e-6) / 1e12 / 8.0, 4), "weight_bytes": wbytes,
            "plan": [{k: st[k] for k in ("path", "ta", "tb", "wpi", "ksl", "S")} for st in ch.describe()["stages"]]}


def bench_chain(args):
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    dev = torch.device("cuda:0")
    M, L, d, q, dff = args.chain_m, 36, 4096, 4096, 12288
    wl = chain_weights(dev, L, d, q, dff)
    X0 = synth.to_torch_bf16(synth.normal_bf16(synth.seed_for(5, 0, 0), M, d), dev)
    flags = (sg.F_KCHUNK if args.chain_kchunk else 0) | (sg.F_LAUNCH_PER_STAGE if args.chain_per_stage else 0)
    ch = sg.LayerChain(M, L, d, q, dff, flags=flags, tn=args.chain_tn)
    ws = ch.new_workspace()
    Y = torch.empty((M, d), dtype=torch.float32, device=dev)
    wbytes = L * 2 * (q * d + d * q + 2 * dff * d + d * dff)
    cols = [[w[i] for w in wl] for i in range(4)]
    if args.copy_calibration:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        ch(X0, *cols, Y, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        ch(X0, *cols, Y, ws)
        ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rc = ch.status(ws)
    if rc:
        raise sg.SgemmError(rc, "chain status")
    ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    avg = sum(ts) / len(ts)
    value = wbytes / (wall / args.steps) / 1e9
    achieved = wbytes / (avg * 1e-6) / 1e9
    out = {
        "metric": "achieved HBM GB/s (weight bytes) and us per decode GEMM, M=1-64 bf16",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"persistent_chain_36_layers_m{M}", "M": M, "layers": L, "d_model": d,
                   "q_cols": q, "d_ff": dff, "weight_bytes_per_step": wbytes, "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "kernel": "k_chain", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(f"chain_m{M}_36l"), "algorithmic_bytes_per_launch": wbytes,
                     "avg_launch_us": round(avg, 2)},
        "chain_us": {"median": round(ts[len(ts) // 2], 2), "min": round(ts[0], 2), "max": round(ts[-1], 2)},
        "plan": [{k: st[k] for k in ("path", "ta", "tb", "waves", "TN", "ksl", "S", "KS", "items")}
                 for st in ch.describe()["stages"]],
    }
    if not args.no_cpu:
        layer_w = [synth.from_torch_bf16(wl[0][i]) for i in range(4)]
        out["cpu_baseline"] = cpu_baseline_chain(M, synth.from_torch_bf16(X0), layer_w)
    return out


def cpu_baseline_decoder(M, x_bits, wn, layer_w, kc, vc, Hq, Hkv):
    """The oracle's decoder layer (RMSNorm, QKV, grouped-query decode
    attention, O with residual, RMSNorm, gate_up with SiLU gate, down with
    residual) on the host cores, repeated on layer 0 for about 10 s."""
    import oracle

    t0 = time.perf_counter()
    reps = 0
    nbytes = 0
    step_bytes = sum(2 * w.size for w in layer_w) + 2 * kc.size + 2 * vc.size
    while True:
        oracle.decoder_layer(x_bits, wn[0], layer_w[0], kc, vc, layer_w[1], wn[1], layer_w[2], layer_w[3], Hq, Hkv)
        nbytes += step_bytes
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 2000:
            break
    dt = time.perf_counter() - t0
    return dict({"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                 "kind": "oracle",
                 "sample": "%d decoder layers (%.1f s) on layer 0's weights, norms, KV cache and input: every "
                           "output, M=%d, double accumulation" % (reps, dt, M)}, **host_cpu())


def bench_decoder(args):
    import math

    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    dev = torch.device("cuda:0")
    M, L, d, dff, Hq, Hkv, hd, T = args.chain_m, 36, 4096, 12288, 32, 8, 128, args.decoder_ctx
    q, kv = Hq * hd, Hkv * hd
    shapes = [(q + 2 * kv, d), (d, q), (2 * dff, d), (d, dff)]
    wl = [[synth.uniform_bf16_torch(synth.seed_for(6, l, 1 + i), r, c, synth.weight_scale(c), dev)
           for i, (r, c) in enumerate(shapes)] for l in range(L)]
    wn_bits = synth.f32_to_bf16_bits(1.0 + synth.bf16_bits_to_f32(
        synth.uniform_bf16(synth.seed_for(6, 0, 7), L * 2, d, 0.25))).reshape(L, 2, d)
    Wn = synth.to_torch_bf16(wn_bits, dev)
    n = L * M * Hkv * T
    Kc = synth.uniform_bf16_torch(synth.seed_for(6, 0, 8), n, hd, math.sqrt(3.0), dev).view(L, M, Hkv, T, hd)
    Vc = synth.uniform_bf16_torch(synth.seed_for(6, 0, 9), n, hd, math.sqrt(3.0), dev).view(L, M, Hkv, T, hd)
    X0 = synth.to_torch_bf16(synth.normal_bf16(synth.seed_for(6, 0, synth.T_X), M, d), dev)
    dec = sg.Decoder(M, L, d, dff, Hq, Hkv, hd, T)
    ws = dec.new_workspace()
    Y = torch.empty((M, d), dtype=torch.float32, device=dev)
    cols = [[w[i] for w in wl] for i in range(4)]
    wbytes = L * sum(2 * r * c for r, c in shapes)
    kvbytes = 2 * 2 * n * hd
    nbytes = wbytes + kvbytes
    if args.copy_calibration:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        dec(X0, Wn, *cols, Kc, Vc, Y, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        dec(X0, Wn, *cols, Kc, Vc, Y, ws)
        ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rc = dec.status(ws)
    if rc:
        raise sg.SgemmError(rc, "decoder status")
    ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    avg = sum(ts) / len(ts)
    achieved = nbytes / (avg * 1e-6) / 1e9
    out = {
        "metric": "achieved HBM GB/s (weight and KV-cache bytes), whole decoder layer chain, bf16",
        "value": round(nbytes / (wall / args.steps) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decoder_36_layers_m{M}_ctx{T}", "M": M, "layers": L, "d_model": d, "d_ff": dff,
                   "heads": Hq, "kv_heads": Hkv, "head_dim": hd, "ctx": T, "weight_bytes_per_step": wbytes,
                   "kv_cache_bytes_per_step": kvbytes, "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "kernel": "k_decoder", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(f"decoder_m{M}_ctx{T}_36l"), "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(avg, 2)},
        "decoder_us": {"median": round(ts[len(ts) // 2], 2), "min": round(ts[0], 2), "max": round(ts[-1], 2)},
        "plan": [{k: st[k] for k in ("path", "ta", "tb", "waves", "TN", "ksl", "S", "KS", "items")}
                 for st in dec.describe()["stages"]],
    }
    if not args.no_cpu:
        lw = [synth.from_torch_bf16(wl[0][i]) for i in range(4)]
        kc0 = synth.from_torch_bf16(Kc[0].reshape(-1, hd)).reshape(M, Hkv, T, hd)
        vc0 = synth.from_torch_bf16(Vc[0].reshape(-1, hd)).reshape(M, Hkv, T, hd)
        out["cpu_baseline"] = cpu_baseline_decoder(M, synth.from_torch_bf16(X0), wn_bits[0], lw, kc0, vc0, Hq, Hkv)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["proj", "chain", "decoder"], default="proj")
    ap.add_argument("--chain-m", type=int, default=64, help="rows of the chain and decoder workloads (1-64)")
    ap.add_argument("--decoder-ctx", type=int, default=1024, help="decoder workload: cached positions per sequence")
    ap.add_argument("--chain-per-stage", action="store_true",
                    help="chain workload: one launch per projection stage (for per-stage counters)")
    ap.add_argument("--chain-kchunk", action="store_true",
                    help="chain workload with every stage on the K-chunked MFMA path (M = 17-32)")
    ap.add_argument("--chain-tn", type=int, default=0, help="chain workload: tile width override (0 = planner)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-configuration table (all GEMM shapes, the 36-layer chain)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy first (counter calibration for --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the per-GPU shard of a "
              "tensor-parallel layout is the same kernel at a narrower shape); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    out = {"proj": bench_proj, "chain": bench_chain, "decoder": bench_decoder}[args.workload](args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
