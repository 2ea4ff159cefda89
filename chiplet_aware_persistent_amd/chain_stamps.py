"""Where the 36-layer chain's time goes, from its per-workgroup stage stamps.

With SGEMM_F_STAMPS every workgroup records the wall clock (100 MHz) when
it is released into a stage (after its wait) and when its last wave ends
the stage.  For every stage after the first this prints, averaged over the
36 layers per projection (Q, O, gate_up, down), in microseconds:

- release: first start of the stage minus the last end of the stage before
  (the barrier's latency as seen by the earliest workgroup);
- skew: last start minus first start;
- med_start: median start minus first start;
- work_med: median over workgroups of end minus own start;
- tail: last end minus median end;
- span: last end minus first start.

    python -m chiplet_aware_persistent_amd.chain_stamps [--m 1 16 64] [--modes default scheduler]
    python -m chiplet_aware_persistent_amd.chain_stamps --m 1 64 --decoder-ctx 1024

Weights and input as in the chain benchmark (distinct seeded
U(-1/sqrt(K), 1/sqrt(K)) bf16 per layer, d = q = 4096, d_ff = 12288).  Each
mode runs 3 warm-up calls, then one call timed with HIP events whose stamps
are analysed.  In scheduler mode the scheduler workgroups (slot 0 of each
XCD, workgroups 0..7) run no stage and are left out.  One JSON line per
(M, mode, projection).
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
STAGES = ("Q", "O", "gate_up", "down")


DECODER_STAGES = ("QKV", "attention", "O", "gate_up", "down")


def stage_breakdown(st, stages=STAGES):
    """st: [workgroups][events][2] start/end stamps in microseconds.  Returns
    {stage: [release, skew, med_start, work_med, tail, span]} averaged over
    the events of that stage (the first event excluded)."""
    import numpy as np

    acc = {n: [] for n in stages}
    for e in range(1, st.shape[1]):
        prev_end = st[:, e - 1, 1]
        s0, s1 = st[:, e, 0], st[:, e, 1]
        acc[stages[e % len(stages)]].append([s0.min() - prev_end.max(), s0.max() - s0.min(), np.median(s0) - s0.min(),
                                   np.median(s1 - s0), s1.max() - np.median(s1), s1.max() - s0.min()])
    return {n: np.mean(np.array(v), axis=0).tolist() for n, v in acc.items() if v}


def main():
    import numpy as np
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    modes = {"default": 0, "scheduler": sg.F_SCHEDULER, "poll_leader": sg.F_POLL_LEADER}
    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, nargs="+", default=[1, 16, 64])
    ap.add_argument("--modes", nargs="+", default=["default", "scheduler"], choices=sorted(modes))
    ap.add_argument("--decoder-ctx", type=int, default=-1,
                    help="time the whole decoder layer instead (cached positions; 5 stages per layer)")
    a = ap.parse_args()
    if a.decoder_ctx >= 0:
        return decoder_main(a)
    dev = torch.device("cuda:0")
    d, q, dff = D_MODEL, Q_COLS, D_FF
    wl = []
    for l in range(LAYERS):
        wl.append([synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WQ), q, d, synth.weight_scale(d), dev),
                   synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WO), d, q, synth.weight_scale(q), dev),
                   synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WGU), 2 * dff, d, synth.weight_scale(d), dev),
                   synth.uniform_bf16_torch(synth.seed_for(5, l, synth.T_WDOWN), d, dff, synth.weight_scale(dff), dev)])
    cols = [[w[i] for w in wl] for i in range(4)]
    for M in a.m:
        X0 = synth.to_torch_bf16(synth.normal_bf16(synth.seed_for(5, 0, synth.T_X), M, d), dev)
        for name in a.modes:
            flags = modes[name]
            ch = sg.LayerChain(M, LAYERS, d, q, dff, flags=sg.F_STAMPS | flags)
            ws = ch.new_workspace()
            Y = torch.empty((M, d), dtype=torch.float32, device=dev)
            for _ in range(3):
                ch(X0, *cols, Y, ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ch(X0, *cols, Y, ws)
            e1.record()
            torch.cuda.synchronize()
            rc = ch.status(ws)
            if rc != sg.OK:
                raise RuntimeError("chain status %s (M=%d, %s)" % (sg.status_string(rc), M, name))
            info = ch.describe()
            E, G, off = 4 * LAYERS, info["grid"], info["stamps_offset"]
            st = ws[off:off + G * E * 16].view(torch.int64).view(G, E, 2).cpu().numpy().astype(np.float64) / 100.0
            if flags & sg.F_SCHEDULER:
                st = st[8:]
            us = e0.elapsed_time(e1) * 1e3
            for proj, v in stage_breakdown(st).items():
                print(json.dumps({"M": M, "mode": name, "chain_us": round(us, 1), "projection": proj,
                                  "release": round(v[0], 2), "skew": round(v[1], 2), "med_start": round(v[2], 2),
                                  "work_med": round(v[3], 2), "tail": round(v[4], 2), "span": round(v[5], 2)}),
                      flush=True)


def decoder_main(a):
    """Stage stamps of the decoder layer (QKV with the attention norm,
    attention, O with the residual, gate_up with the MLP norm, down with the
    residual), 36 layers, weights and KV cache as in the decoder benchmark."""
    import math

    import numpy as np
    import torch

    import chiplet_aware_persistent_amd as sg
    import synth

    dev = torch.device("cuda:0")
    L, d, dff, Hq, Hkv, hd, T = LAYERS, D_MODEL, D_FF, 32, 8, 128, a.decoder_ctx
    q, kv = Hq * hd, Hkv * hd
    shapes = [(q + 2 * kv, d), (d, q), (2 * dff, d), (d, dff)]
    wl = [[synth.uniform_bf16_torch(synth.seed_for(6, l, 1 + i), r, c, synth.weight_scale(c), dev)
           for i, (r, c) in enumerate(shapes)] for l in range(L)]
    cols = [[w[i] for w in wl] for i in range(4)]
    wn = synth.f32_to_bf16_bits(1.0 + synth.bf16_bits_to_f32(
        synth.uniform_bf16(synth.seed_for(6, 0, 7), L * 2, d, 0.25))).reshape(L, 2, d)
    Wn = synth.to_torch_bf16(wn, dev)
    for M in a.m:
        n = L * M * Hkv * max(T, 1)
        Kc = synth.uniform_bf16_torch(synth.seed_for(6, 0, 8), n, hd, math.sqrt(3.0), dev)
        Vc = synth.uniform_bf16_torch(synth.seed_for(6, 0, 9), n, hd, math.sqrt(3.0), dev)
        Kc = Kc[: L * M * Hkv * T].view(L, M, Hkv, T, hd)
        Vc = Vc[: L * M * Hkv * T].view(L, M, Hkv, T, hd)
        X0 = synth.to_torch_bf16(synth.normal_bf16(synth.seed_for(6, 0, synth.T_X), M, d), dev)
        dec = sg.Decoder(M, L, d, dff, Hq, Hkv, hd, T, flags=sg.F_STAMPS)
        ws = dec.new_workspace()
        Y = torch.empty((M, d), dtype=torch.float32, device=dev)
        for _ in range(3):
            dec(X0, Wn, *cols, Kc, Vc, Y, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dec(X0, Wn, *cols, Kc, Vc, Y, ws)
        e1.record()
        torch.cuda.synchronize()
        rc = dec.status(ws)
        if rc != sg.OK:
            raise RuntimeError("decoder status %s (M=%d)" % (sg.status_string(rc), M))
        info = dec.describe()
        E, G, off = 5 * L, info["grid"], info["stamps_offset"]
        st = ws[off:off + G * E * 16].view(torch.int64).view(G, E, 2).cpu().numpy().astype(np.float64) / 100.0
        us = e0.elapsed_time(e1) * 1e3
        for stage, v in stage_breakdown(st, DECODER_STAGES).items():
            print(json.dumps({"M": M, "mode": "decoder", "ctx": T, "decoder_us": round(us, 1), "stage": stage,
                              "release": round(v[0], 2), "skew": round(v[1], 2), "med_start": round(v[2], 2),
                              "work_med": round(v[3], 2), "tail": round(v[4], 2), "span": round(v[5], 2)}),
                  flush=True)


if __name__ == "__main__":
    main()
