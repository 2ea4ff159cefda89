"""GPU parity of the whole decoder layer (decoder_run: RMSNorm, QKV, grouped-
query decode attention, O with the residual, RMSNorm, gate_up with the SiLU
gate, down with the residual, all layers in one persistent launch) against the
CPU oracle, stage by stage on the GPU's own input to each stage.

Bounds.  A projection gets the stated 2e-3 * sum|x w| + 1e-6 (+ one bf16 ulp
of a bf16 output).  Where the projection's input is a normalised row that the
GPU forms in LDS (QKV, gate_up), the GPU's bf16 of x * rstd * w may differ by
one ulp from the oracle's, which adds sum_k ulp(n_k) |w_k|.  The attention
output gets one bf16 ulp plus 1e-3 * sum_t p_t |v_t| (fp32 scores, exp and
sums against the oracle's double) plus 1e-6.  The SiLU gate gets the chain's
propagated bound.
"""
import math

import numpy as np
import pytest

import chiplet_aware_persistent_amd as sg
import oracle
import synth
from helpers import device_tensor_bf16, host_bits, report

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
special = pytest.importorskip("scipy.special")


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def make_decoder(M, L, d, dff, Hq, Hkv, hd, T, seed, dev, weights_on_device=False):
    q, kv = Hq * hd, Hkv * hd
    shapes = [(q + 2 * kv, d), (d, q), (2 * dff, d), (d, dff)]
    seeds = [[seed + 16 * l + i for i in range(1, 5)] for l in range(L)]
    if weights_on_device:
        dl = [[synth.uniform_bf16_torch(seeds[l][i], shapes[i][0], shapes[i][1], synth.weight_scale(shapes[i][1]),
                                        dev) for i in range(4)] for l in range(L)]
        hl = None
    else:
        hl = [[synth.uniform_bf16(seeds[l][i], shapes[i][0], shapes[i][1], synth.weight_scale(shapes[i][1]))
               for i in range(4)] for l in range(L)]
        dl = [[device_tensor_bf16(w, dev) for w in ws] for ws in hl]
    wn = synth.f32_to_bf16_bits(1.0 + synth.bf16_bits_to_f32(synth.uniform_bf16(seed + 7, L * 2, d, 0.25)))
    wn = wn.reshape(L, 2, d)
    n = L * M * Hkv * T * hd
    kc = synth.uniform_bf16_torch(seed + 8, max(n // hd, 1), hd, math.sqrt(3.0), dev)[: n // hd]
    vc = synth.uniform_bf16_torch(seed + 9, max(n // hd, 1), hd, math.sqrt(3.0), dev)[: n // hd]
    kc = kc.reshape(L, M, Hkv, T, hd)
    vc = vc.reshape(L, M, Hkv, T, hd)
    x0 = synth.normal_bf16(seed, M, d)
    return x0, wn, hl, dl, kc, vc


def run_decoder(dec, X0, Wn, dl, Kc, Vc, ws=None):
    Y = torch.empty((dec.M, dec.d), dtype=torch.float32, device=X0.device)
    Yb = torch.empty((dec.M, dec.d), dtype=torch.bfloat16, device=X0.device)
    if ws is None:
        ws = dec.new_workspace()
    dec(X0, Wn, [w[0] for w in dl], [w[1] for w in dl], [w[2] for w in dl], [w[3] for w in dl], Kc, Vc, Y, ws,
        Y_bf16=Yb)
    return dec.status(ws), Y, Yb, ws


def _normed_gemm_bound(n_bits, w_bits):
    """(y_ref, bound) of n . w^T where n is a normalised bf16 row the GPU
    formed itself (one ulp apart at most)."""
    y_ref, absdot = oracle.gemm(n_bits, w_bits)
    prop = oracle.bf16_ulp(f64(n_bits)) @ np.abs(f64(w_bits)).T
    return y_ref, oracle.REL_TOL * absdot + prop + oracle.ABS_TOL


def _attn_weight_abs(q_bits, kc, vc, kn, vn, Hq, Hkv):
    """sum_t p_t |v_t| per output element (double), for the attention bound."""
    M, _, T, hd = kc.shape
    Q = f64(q_bits).reshape(M, Hq, hd)
    K = np.concatenate([f64(kc), f64(kn).reshape(M, Hkv, 1, hd)], axis=2)
    V = np.abs(np.concatenate([f64(vc), f64(vn).reshape(M, Hkv, 1, hd)], axis=2))
    out = np.empty((M, Hq, hd))
    for m in range(M):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            p = special.softmax(K[m, g] @ Q[m, h] / math.sqrt(hd))
            out[m, h] = p @ V[m, g]
    return out.reshape(M, Hq * hd)


def check_decoder(dec, ws, x0, wn, layer_w, kc, vc, Y, Yb, name=None):
    """Every stage of every layer against the oracle on the GPU's own input."""
    q, kv, dff = dec.q, dec.kv, dec.dff
    x_in = x0
    worst = {"qkv": 0.0, "o": 0.0, "x1": 0.0, "a": 0.0, "x_out": 0.0, "y_f32": 0.0}

    def take(key, err, b, l):
        r = float(np.max(err / b)) if err.size else 0.0
        assert r <= 1.0, (l, key, r)
        worst[key] = max(worst[key], r)

    kch, vch = host_bits(kc.reshape(-1, dec.hd)), host_bits(vc.reshape(-1, dec.hd))
    kch = kch.reshape(tuple(kc.shape))
    vch = vch.reshape(tuple(vc.shape))
    for l in range(dec.n_layers):
        wqkv, wo, wgu, wdown = layer_w(l)
        got = [host_bits(dec.activation(ws, l, w)) for w in range(5)]
        # QKV on the normalised input
        n1 = oracle.rmsnorm(x_in, wn[l, 0])
        y, b = _normed_gemm_bound(n1, wqkv)
        take("qkv", np.abs(f64(got[0]) - y), b + oracle.bf16_ulp(y), l)
        # attention on the GPU's own q, k, v
        qg, kg, vg = got[0][:, :q], got[0][:, q:q + kv], got[0][:, q + kv:]
        o_ref = f64(oracle.gqa_decode(qg, kch[l], vch[l], kg, vg, dec.Hq, dec.Hkv))
        ba = oracle.bf16_ulp(o_ref) + 1e-3 * _attn_weight_abs(qg, kch[l], vch[l], kg, vg, dec.Hq, dec.Hkv) + 1e-6
        take("o", np.abs(f64(got[1]) - o_ref), ba, l)
        # O + residual
        y, ad = oracle.gemm(got[1], wo)
        x1_ref = f64(oracle.residual(x_in, y))
        take("x1", np.abs(f64(got[2]) - x1_ref), oracle.bound(ad) + oracle.bf16_ulp(x1_ref), l)
        # gate_up on the normalised x1, SiLU gate
        n2 = oracle.rmsnorm(got[2], wn[l, 1])
        gu, bgu = _normed_gemm_bound(n2, wgu)
        g32, u32 = gu[:, :dff].astype(np.float32), gu[:, dff:].astype(np.float32)
        a_ref = f64(oracle.silu_gate(g32, u32))
        bg, bu = bgu[:, :dff], bgu[:, dff:]
        g64, u64 = g32.astype(np.float64), u32.astype(np.float64)
        bsa = (1.1 * bg * (np.abs(u64) + bu) + (np.abs(g64 * special.expit(g64)) + 1.1 * bg) * bu
               + 2.0 ** -20 * np.abs(a_ref) + oracle.bf16_ulp(a_ref))
        take("a", np.abs(f64(got[3]) - a_ref), bsa, l)
        # down + residual
        y, ad = oracle.gemm(got[3], wdown)
        xo_ref = f64(oracle.residual(got[2], y))
        take("x_out", np.abs(f64(got[4]) - xo_ref), oracle.bound(ad) + oracle.bf16_ulp(xo_ref), l)
        if l == dec.n_layers - 1:
            yref = f64(got[2]) + y
            take("y_f32", np.abs(Y.cpu().numpy().astype(np.float64) - yref),
                 oracle.bound(ad) + 2.0 ** -23 * np.abs(yref), l)
            assert np.array_equal(host_bits(Yb), got[4])
        x_in = got[4]
    if name:
        report(name, max(worst.values()), per_stage=worst)
    return worst


SMALL = [(1, 0), (1, 5), (2, 70), (5, 130), (16, 64), (33, 1), (64, 200), (3, 0), (17, 127)]


@pytest.mark.parametrize("M,T", SMALL)
def test_decoder_small_parity(cuda_device, M, T):
    """Two layers, d = 256, d_ff = 384, 8 query / 2 key-value heads of 128:
    dot2 stages at M <= 2, MFMA above; cached lengths that leave 1..64
    positions in the last attention chunk, and none."""
    L, d, dff, Hq, Hkv, hd = 2, 256, 384, 8, 2, 128
    x0, wn, hl, dl, kc, vc = make_decoder(M, L, d, dff, Hq, Hkv, hd, T, 0x8000 + 16 * M + T, cuda_device)
    dec = sg.Decoder(M, L, d, dff, Hq, Hkv, hd, T)
    Wn = device_tensor_bf16(wn.reshape(L, 2 * d), cuda_device).reshape(L, 2, d)
    rc, Y, Yb, ws = run_decoder(dec, device_tensor_bf16(x0, cuda_device), Wn, dl, kc, vc)
    assert rc == sg.OK, sg.status_string(rc)
    check_decoder(dec, ws, x0, wn, lambda l: hl[l], kc, vc, Y, Yb)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("M", [1, 16, 64])
def test_decoder_qwen3_8b_shapes(cuda_device, M):
    """Qwen3-8B-shaped layers (d = 4096, d_ff = 12288, 32 query / 8 key-value
    heads of 128, 1024 cached positions), two layers, every output element of
    every stage against the oracle."""
    L, d, dff, Hq, Hkv, hd, T = 2, 4096, 12288, 32, 8, 128, 1024
    x0, wn, _, dl, kc, vc = make_decoder(M, L, d, dff, Hq, Hkv, hd, T, 0x9000 + M, cuda_device,
                                         weights_on_device=True)
    dec = sg.Decoder(M, L, d, dff, Hq, Hkv, hd, T)
    Wn = device_tensor_bf16(wn.reshape(L, 2 * d), cuda_device).reshape(L, 2, d)
    rc, Y, Yb, ws = run_decoder(dec, device_tensor_bf16(x0, cuda_device), Wn, dl, kc, vc)
    assert rc == sg.OK, sg.status_string(rc)
    check_decoder(dec, ws, x0, wn, lambda l: [host_bits(w) for w in dl[l]], kc, vc, Y, Yb,
                  name="decoder qwen3-8b shapes m%d" % M)


def test_decoder_repeatable_and_graph_replays(cuda_device):
    """Repeated runs on one workspace and HIP graph replays give bitwise the
    same output (attention combine and split-K counters reset themselves)."""
    M, L, d, dff, Hq, Hkv, hd, T = 16, 3, 512, 768, 16, 4, 128, 300
    x0, wn, hl, dl, kc, vc = make_decoder(M, L, d, dff, Hq, Hkv, hd, T, 0xA000, cuda_device)
    dec = sg.Decoder(M, L, d, dff, Hq, Hkv, hd, T)
    Wn = device_tensor_bf16(wn.reshape(L, 2 * d), cuda_device).reshape(L, 2, d)
    X0 = device_tensor_bf16(x0, cuda_device)
    rc, Ye, Ybe, ws = run_decoder(dec, X0, Wn, dl, kc, vc)
    assert rc == sg.OK
    check_decoder(dec, ws, x0, wn, lambda l: hl[l], kc, vc, Ye, Ybe)
    for r in range(3):
        rc, Y2, _, ws = run_decoder(dec, X0, Wn, dl, kc, vc, ws)
        assert rc == sg.OK and torch.equal(Y2, Ye), r
    cols = [[w[i] for w in dl] for i in range(4)]
    Y, Yb = torch.empty_like(Ye), torch.empty_like(Ybe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec(X0, Wn, *cols, kc, vc, Y, ws, Y_bf16=Yb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec(X0, Wn, *cols, kc, vc, Y, ws, Y_bf16=Yb)
    for r in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert dec.status(ws) == sg.OK, r
        assert torch.equal(Y, Ye) and torch.equal(Yb, Ybe), r
