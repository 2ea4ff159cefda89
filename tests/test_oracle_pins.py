"""Pins of the CPU oracle and of the seeded generator against facts that do not
come from the oracle itself: a published generator test vector, exact rational
arithmetic, integer arithmetic, closed forms, a library matmul and library
special functions.  Each test is chosen so that a plausible slip in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a wrong rounding
rule, swapped gate/up halves) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ generator
def test_splitmix64_published_vector():
    g = json.load(open(os.path.join(GOLD, "splitmix64_seed1234567.json")))
    got = synth.splitmix64_sequence(g["state"], len(g["outputs"]))
    assert got == [int(v) for v in g["outputs"]]


def test_counter_stream_equals_sequential_generator():
    seed = synth.seed_for(3, 2, synth.T_WO)
    k = synth.key(seed)
    seq = synth.splitmix64_sequence(k, 300)
    vec = synth.stream_u64(seed, 0, 300)
    assert [int(v) for v in vec] == seq
    # any slice can be drawn on its own
    assert [int(v) for v in synth.stream_u64(seed, 123, 10)] == seq[123:133]


def test_torch_generator_matches_numpy_cpu():
    torch = pytest.importorskip("torch")
    seed, a = synth.seed_for(1, 0, synth.T_WGU), synth.weight_scale(4096)
    ref = synth.uniform_bf16(seed, 37, 129, a)
    t = synth.uniform_bf16_torch(seed, 37, 129, a, device="cpu", chunk_elems=1000)
    assert np.array_equal(synth.from_torch_bf16(t), ref)
    rows = synth.uniform_bf16_rows(seed, 129, a, [0, 5, 36])
    assert np.array_equal(rows, ref[[0, 5, 36]])


def test_distributions():
    a = synth.weight_scale(1024)
    w = synth.bf16_bits_to_f32(synth.uniform_bf16(11, 256, 1024, a)).astype(np.float64)
    assert np.all(np.abs(w) <= a * (1 + 2 ** -8))
    assert abs(w.mean()) < 0.01 * a
    assert abs(w.var() / (a * a / 3.0) - 1.0) < 0.02
    x = synth.bf16_bits_to_f32(synth.normal_bf16(12, 64, 4096)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


# ------------------------------------------------------------- bf16 rounding
TRICKY = [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
          -(1.0 + 2 ** -8), 3.4e38, 3.3895314e38, 1e-40, -1e-40, 2 ** -133, 2 ** -126,
          float("inf"), -float("inf"), 65504.0, 0.1, -0.3333333, 1.99609375, 255.5]


@pytest.mark.parametrize("impl", ["oracle", "synth"])
def test_bf16_rne_against_torch(impl):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    vals = np.concatenate([np.array(TRICKY, np.float32),
                           rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                           rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    vals = vals[np.isfinite(vals) | np.isinf(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_f32(vals) if impl == "oracle" else synth.f32_to_bf16_bits(vals)
    assert np.array_equal(got, ref)
    # ties go to even
    one_tie = np.array([1.0 + 2 ** -8], np.float32)
    assert (oracle.bf16_from_f32(one_tie)[0], synth.f32_to_bf16_bits(one_tie)[0]) == (0x3F80, 0x3F80)


def test_bf16_nan_stays_nan():
    nan = np.array([float("nan")], np.float32)
    b = int(oracle.bf16_from_f32(nan)[0])
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


# ------------------------------------------------------------------- GEMM
def _exact(x_bits, w_bits):
    xf = synth.bf16_bits_to_f32(x_bits)
    wf = synth.bf16_bits_to_f32(w_bits)
    M, K = xf.shape
    N = wf.shape[0]
    out = [[sum((Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(K)), Fraction(0))
            for n in range(N)] for m in range(M)]
    return out, xf.astype(np.float64), wf.astype(np.float64)


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (1, 8, 3), (3, 5, 7), (8, 8, 8), (2, 7, 1), (7, 3, 8)])
def test_bruteforce_tiny_vs_exact_rationals(M, K, N):
    x = synth.normal_bf16(100 + M, M, K)
    w = synth.uniform_bf16(200 + N, N, K, synth.weight_scale(K))
    y, a = oracle.gemm(x, w)
    ex, xf, wf = _exact(x, w)
    absdot = np.abs(xf)[:, None, :] * np.abs(wf)[None, :, :]
    for m in range(M):
        for n in range(N):
            s = absdot[m, n].sum()
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= Fraction(K * 2.0 ** -52 * s + 1e-300)
            assert abs(a[m, n] - s) <= K * 2.0 ** -52 * s


def test_against_numpy_float64_matmul():
    x = synth.normal_bf16(1, 5, 300)
    w = synth.uniform_bf16(2, 77, 300, synth.weight_scale(300))
    y, a = oracle.gemm(x, w)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    np.testing.assert_allclose(y, xf @ wf.T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(a, np.abs(xf) @ np.abs(wf).T, rtol=1e-14)


def test_integer_inputs_are_exact():
    x = synth.int_bf16(3, 7, 1000, -3, 3)
    w = synth.int_bf16(4, 33, 1000, -3, 3)
    y, _ = oracle.gemm(x, w)
    xi = synth.bf16_bits_to_f32(x).astype(np.int64)
    wi = synth.bf16_bits_to_f32(w).astype(np.int64)
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))
    assert np.any(y < 0) and np.any(y > 0)


@pytest.mark.parametrize("K", [1024, 4096, 7168, 12288])
def test_all_ones_gives_K(K):
    one = synth.f32_to_bf16_bits(np.ones((2, K), np.float32))
    w = synth.f32_to_bf16_bits(np.ones((3, K), np.float32))
    y, a = oracle.gemm(one, w)
    assert np.all(y == K) and np.all(a == K)


def test_one_hot_weights_copy_columns():
    M, K, N = 3, 40, 17
    rng = np.random.default_rng(0)
    perm = rng.permutation(K)[:N]  # column n of Y copies column perm[n] of X
    w = np.zeros((N, K), np.float32)
    w[np.arange(N), perm] = 1.0
    x = synth.normal_bf16(9, M, K)
    y, _ = oracle.gemm(x, synth.f32_to_bf16_bits(w))
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    assert np.array_equal(y, xf[:, perm])


def test_power_of_two_scaling_is_exact():
    x = synth.normal_bf16(21, 4, 512)
    w = synth.uniform_bf16(22, 9, 512, synth.weight_scale(512))
    y, _ = oracle.gemm(x, w)
    xs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(2.0 ** 5))
    ws = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(w) * np.float32(2.0 ** -3))
    y2, _ = oracle.gemm(xs, ws)
    assert np.array_equal(y2, y * 4.0)


def test_linearity_with_disjoint_support():
    K = 600
    x = synth.normal_bf16(31, 3, K)
    w = synth.uniform_bf16(32, 11, K, synth.weight_scale(K))
    mask = (np.arange(K) % 3) == 0
    x1 = np.where(mask[None, :], x, 0).astype(np.uint16)
    x2 = np.where(mask[None, :], 0, x).astype(np.uint16)
    y, a = oracle.gemm(x, w)
    y1, _ = oracle.gemm(x1, w)
    y2, _ = oracle.gemm(x2, w)
    assert np.all(np.abs(y - (y1 + y2)) <= 1e-14 * a)


# ------------------------------------------------------------------- SiLU
def test_silu_identities():
    scipy_special = pytest.importorskip("scipy.special")
    assert oracle.silu(0.0) == 0.0
    for v in [0.1, 0.5, 1.0, 2.5, 7.0, 20.0]:
        assert abs((oracle.silu(v) - oracle.silu(-v)) - v) <= 1e-15 * max(1.0, v)
        assert abs(oracle.silu(v) - v * scipy_special.expit(v)) <= 1e-15 * max(1.0, v)
    assert oracle.silu(50.0) == 50.0
    assert 0 > oracle.silu(-50.0) > -1e-19


def test_silu_gate_array_matches_closed_forms():
    """The array form of the chain's SiLU gate: zero gate or zero up gives 0,
    silu(g) -> g for large g (so a = bf16(g u)), the odd-part identity
    silu(g) - silu(-g) = g on paired inputs, and agreement with
    g * expit(g) * u rounded through fp32 to bf16 (within one bf16 ulp, the
    rounding-order difference)."""
    special = pytest.importorskip("scipy.special")
    g = np.array([0.0, 0.0, 3.0, 40.0, 60.0, -60.0, 1.5], np.float32)
    u = np.array([5.0, -2.0, 0.0, 0.5, -3.0, 7.0, 1.0], np.float32)
    a = synth.bf16_bits_to_f32(oracle.silu_gate(g, u)).astype(np.float64)
    assert a[0] == 0.0 and a[1] == 0.0 and a[2] == 0.0
    assert a[3] == 20.0 and a[4] == -180.0
    tiny = -60.0 * math.exp(-60.0) / (1.0 + math.exp(-60.0)) * 7.0   # silu(-60) * 7, about -3.7e-24
    assert abs(a[5] - tiny) <= oracle.bf16_ulp(tiny)
    rng = np.random.default_rng(5)
    gg = rng.normal(size=(7, 33)).astype(np.float32)
    uu = rng.normal(size=(7, 33)).astype(np.float32)
    got = synth.bf16_bits_to_f32(oracle.silu_gate(gg, uu)).astype(np.float64)
    ones = np.ones_like(gg)
    pos = synth.bf16_bits_to_f32(oracle.silu_gate(gg, ones)).astype(np.float64)
    neg = synth.bf16_bits_to_f32(oracle.silu_gate(-gg, ones)).astype(np.float64)
    assert np.all(np.abs(pos - neg - gg) <= oracle.bf16_ulp(pos) + oracle.bf16_ulp(neg))
    g64 = gg.astype(np.float64)
    ref = synth.bf16_bits_to_f32(_bits(g64 * special.expit(g64) * uu.astype(np.float64))).astype(np.float64)
    assert np.all(np.abs(got - ref) <= oracle.bf16_ulp(ref))
    assert np.mean(got == ref) > 0.95


# ------------------------------------------------------------------- chain
def _bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


def test_chain_one_hot_layer_reduces_to_silu_gate():
    """Identity Wq/Wo and one-hot gate/up/down rows: x'_i = bf16(silu(x_p) * x_q)."""
    special = pytest.importorskip("scipy.special")
    torch = pytest.importorskip("torch")
    M, d, dff = 4, 8, 5
    p = [3, 0, 7, 2, 5]       # gate column j reads x[p[j]]
    q = [1, 6, 4, 4, 0]       # up column j reads x[q[j]]
    sel = [2, 4, 0, 1, 3, 2, 0, 4]  # output i copies a[sel[i]]
    eye = np.eye(d, dtype=np.float32)
    wgu = np.zeros((2 * dff, d), np.float32)
    wgu[np.arange(dff), p] = 1.0
    wgu[dff + np.arange(dff), q] = 1.0
    wdown = np.zeros((d, dff), np.float32)
    wdown[np.arange(d), sel] = 1.0
    x = synth.normal_bf16(77, M, d)
    r = oracle.layer(x, _bits(eye), _bits(eye), _bits(wgu), _bits(wdown))
    assert np.array_equal(r["h1"], x) and np.array_equal(r["h2"], x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    g, u = xf[:, p], xf[:, q]
    a_ref = torch.from_numpy((g * special.expit(g) * u).astype(np.float32)).to(torch.bfloat16)
    a_ref = a_ref.view(torch.int16).numpy().view(np.uint16)
    diff = np.abs(r["a"].astype(np.int32) - a_ref.astype(np.int32))
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.9
    assert np.array_equal(r["x_out"], r["a"][:, sel])
    assert np.array_equal(r["y_f32"], synth.bf16_bits_to_f32(r["a"][:, sel]))


def test_chain_small_random_against_numpy_composition():
    special = pytest.importorskip("scipy.special")
    M, d, q, dff = 3, 16, 12, 24
    layers = []
    for l in range(2):
        layers.append((synth.uniform_bf16(500 + l, q, d, synth.weight_scale(d)),
                       synth.uniform_bf16(600 + l, d, q, synth.weight_scale(q)),
                       synth.uniform_bf16(700 + l, 2 * dff, d, synth.weight_scale(d)),
                       synth.uniform_bf16(800 + l, d, dff, synth.weight_scale(dff))))
    x0 = synth.normal_bf16(999, M, d)
    outs = oracle.chain(x0, layers)
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)
    x = f(x0)
    for (wq, wo, wgu, wdown), r in zip(layers, outs):
        h1 = f(_bits(x @ f(wq).T))
        h2 = f(_bits(h1 @ f(wo).T))
        gu = (h2 @ f(wgu).T).astype(np.float32).astype(np.float64)
        g, u = gu[:, :dff], gu[:, dff:]
        a = f(_bits(g * special.expit(g) * u))
        y = a @ f(wdown).T
        for name, ref in [("h1", h1), ("h2", h2), ("a", a)]:
            got = f(r[name])
            assert np.all(np.abs(got - ref) <= oracle.bf16_ulp(ref) * 1.0001), name
        assert np.all(np.abs(r["y_f32"] - y) <= 1e-6 * np.abs(y) + 1e-30)
        x = f(r["x_out"])


def test_tolerance_helpers():
    assert oracle.bf16_ulp(1.0) == 2.0 ** -7
    assert oracle.bf16_ulp(-3.0) == 2.0 ** -6
    b = oracle.bound(np.array([1.0]), y_ref=np.array([1.0]), bf16_out=True)
    assert math.isclose(b[0], 2e-3 + 1e-6 + 2 ** -7)


# ------------------------------------------------------- decoder-layer pieces
def _f(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def test_rmsnorm_constant_row_and_scale_invariance():
    """A constant row c normalises to sign(c) (times the weight); scaling a
    row by a power of two leaves the result unchanged (eps negligible)."""
    d = 64
    w = synth.f32_to_bf16_bits(np.linspace(0.5, 2.0, d).astype(np.float32))
    x = synth.f32_to_bf16_bits(np.array([[3.0] * d, [-0.25] * d], np.float32))
    out = _f(oracle.rmsnorm(x, w, eps=0.0))
    assert np.array_equal(out[0], _f(w)) and np.array_equal(out[1], -_f(w))
    r = synth.normal_bf16(21, 3, 1000)
    w2 = synth.uniform_bf16(22, 1, 1000, 1.0)[0]
    base = oracle.rmsnorm(r, w2, eps=1e-30)
    for a in (-3, 5):
        scaled = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(r) * np.float32(2.0 ** a))
        assert np.array_equal(oracle.rmsnorm(scaled, w2, eps=1e-30), base)


def test_rmsnorm_against_numpy():
    x = synth.normal_bf16(23, 5, 4096)
    w = synth.uniform_bf16(24, 1, 4096, 2.0)[0]
    got = _f(oracle.rmsnorm(x, w))
    xf = _f(x)
    ref = xf / np.sqrt(np.mean(xf ** 2, axis=1, keepdims=True) + oracle.RMS_EPS) * _f(w)[None, :]
    assert np.all(np.abs(got - ref) <= oracle.bf16_ulp(ref))


def _attn_inputs(M, Hq, Hkv, hd, T, seed):
    q = synth.normal_bf16(seed, M, Hq * hd)
    kc = synth.normal_bf16(seed + 1, M * Hkv * T, hd).reshape(M, Hkv, T, hd)
    vc = synth.normal_bf16(seed + 2, M * Hkv * T, hd).reshape(M, Hkv, T, hd)
    kn = synth.normal_bf16(seed + 3, M, Hkv * hd)
    vn = synth.normal_bf16(seed + 4, M, Hkv * hd)
    return q, kc, vc, kn, vn


def test_attention_equal_keys_give_the_mean_of_values():
    """All keys equal (cached and new): uniform weights, the output is the mean
    of the T + 1 values of the query's key/value head."""
    M, Hq, Hkv, hd, T = 2, 8, 2, 16, 9
    q, kc, vc, kn, vn = _attn_inputs(M, Hq, Hkv, hd, T, 31)
    key = synth.normal_bf16(40, 1, hd)[0]
    kc[:] = key
    kn[:] = np.tile(key, Hkv)
    out = _f(oracle.gqa_decode(q, kc, vc, kn, vn, Hq, Hkv)).reshape(M, Hq, hd)
    for m in range(M):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            vals = np.concatenate([_f(vc[m, g]), _f(vn[m].reshape(Hkv, hd)[g])[None, :]])
            ref = vals.mean(axis=0)
            assert np.all(np.abs(out[m, h] - ref) <= oracle.bf16_ulp(ref)), (m, h)


def test_attention_dominant_key_selects_its_value_and_head_groups():
    """One key aligned with a large multiple of the query dominates the
    softmax, so the output is that position's value; value heads filled with
    a constant per key/value head show the grouping h -> h / (Hq / Hkv)."""
    M, Hq, Hkv, hd, T = 1, 8, 4, 32, 6
    q, kc, vc, kn, vn = _attn_inputs(M, Hq, Hkv, hd, T, 51)
    qf = _f(q).reshape(Hq, hd)
    kc[:] = 0
    kn[:] = 0
    for g in range(Hkv):
        # position 3 of key head g: 64 x the first query of its group, others zero
        kc[0, g, 3] = synth.f32_to_bf16_bits((qf[g * (Hq // Hkv)] * 64.0).astype(np.float32))
    out = _f(oracle.gqa_decode(q, kc, vc, kn, vn, Hq, Hkv)).reshape(Hq, hd)
    for g in range(Hkv):
        h = g * (Hq // Hkv)
        assert np.array_equal(out[h], _f(vc[0, g, 3])), h
    vc2 = np.empty_like(vc)
    vn2 = np.empty_like(vn)
    for g in range(Hkv):
        vc2[:, g] = synth.f32_to_bf16_bits(np.float32(0.5 * (g + 1)))
        vn2.reshape(M, Hkv, hd)[:, g] = synth.f32_to_bf16_bits(np.float32(0.5 * (g + 1)))
    out2 = _f(oracle.gqa_decode(q, kc, vc2, kn, vn2, Hq, Hkv)).reshape(Hq, hd)
    for h in range(Hq):
        assert np.all(out2[h] == 0.5 * (h // (Hq // Hkv) + 1)), h


def test_attention_permutation_and_value_scaling():
    """Permuting the cached positions (keys with their values) leaves the
    output unchanged; doubling every value doubles it exactly."""
    M, Hq, Hkv, hd, T = 2, 4, 2, 16, 11
    q, kc, vc, kn, vn = _attn_inputs(M, Hq, Hkv, hd, T, 61)
    base = oracle.gqa_decode(q, kc, vc, kn, vn, Hq, Hkv)
    perm = np.random.default_rng(0).permutation(T)
    got = oracle.gqa_decode(q, kc[:, :, perm], vc[:, :, perm], kn, vn, Hq, Hkv)
    assert np.all(np.abs(_f(got) - _f(base)) <= oracle.bf16_ulp(_f(base)))
    two = lambda b: synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(b) * np.float32(2.0))
    assert np.array_equal(_f(oracle.gqa_decode(q, kc, two(vc), kn, two(vn), Hq, Hkv)), 2.0 * _f(base))


def test_attention_against_numpy_softmax():
    special = pytest.importorskip("scipy.special")
    M, Hq, Hkv, hd, T = 3, 8, 2, 32, 20
    q, kc, vc, kn, vn = _attn_inputs(M, Hq, Hkv, hd, T, 71)
    got = _f(oracle.gqa_decode(q, kc, vc, kn, vn, Hq, Hkv)).reshape(M, Hq, hd)
    K = np.concatenate([_f(kc), _f(kn).reshape(M, Hkv, 1, hd)], axis=2)
    V = np.concatenate([_f(vc), _f(vn).reshape(M, Hkv, 1, hd)], axis=2)
    Q = _f(q).reshape(M, Hq, hd)
    for m in range(M):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            p = special.softmax(K[m, g] @ Q[m, h] / np.sqrt(hd))
            ref = p @ V[m, g]
            assert np.all(np.abs(got[m, h] - ref) <= oracle.bf16_ulp(ref) * 1.0001 + 1e-30), (m, h)


def test_residual_identities():
    x = synth.normal_bf16(81, 4, 50)
    assert np.array_equal(oracle.residual(x, np.zeros((4, 50))), x)
    y = np.random.default_rng(1).normal(size=(4, 50))
    zero = np.zeros((4, 50), np.uint16)
    assert np.array_equal(oracle.residual(zero, y), synth.f32_to_bf16_bits(y.astype(np.float32)))
    # x + f32(y) is one fp32 rounding, then one bf16 rounding
    ref = synth.f32_to_bf16_bits((_f(x) + y.astype(np.float32).astype(np.float64)).astype(np.float32))
    assert np.array_equal(oracle.residual(x, y), ref)


def test_decoder_layer_small_against_numpy_composition():
    special = pytest.importorskip("scipy.special")
    M, d, Hq, Hkv, hd, T, dff = 2, 64, 4, 2, 16, 5, 96
    qc, kvc = Hq * hd, Hkv * hd
    x = synth.normal_bf16(91, M, d)
    w_attn = synth.uniform_bf16(92, 1, d, 2.0)[0]
    w_mlp = synth.uniform_bf16(93, 1, d, 2.0)[0]
    wqkv = synth.uniform_bf16(94, qc + 2 * kvc, d, synth.weight_scale(d))
    wo = synth.uniform_bf16(95, d, qc, synth.weight_scale(qc))
    wgu = synth.uniform_bf16(96, 2 * dff, d, synth.weight_scale(d))
    wdown = synth.uniform_bf16(97, d, dff, synth.weight_scale(dff))
    kc = synth.normal_bf16(98, M * Hkv * T, hd).reshape(M, Hkv, T, hd)
    vc = synth.normal_bf16(99, M * Hkv * T, hd).reshape(M, Hkv, T, hd)
    r = oracle.decoder_layer(x, w_attn, wqkv, kc, vc, wo, w_mlp, wgu, wdown, Hq, Hkv)
    b = lambda v: _f(synth.f32_to_bf16_bits(np.asarray(v, np.float64).astype(np.float32)))
    xf = _f(x)
    n1 = b(xf / np.sqrt(np.mean(xf ** 2, 1, keepdims=True) + oracle.RMS_EPS) * _f(w_attn))
    qkv = b(n1 @ _f(wqkv).T)
    q, k, v = qkv[:, :qc], qkv[:, qc:qc + kvc], qkv[:, qc + kvc:]
    K = np.concatenate([_f(kc), k.reshape(M, Hkv, 1, hd)], axis=2)
    V = np.concatenate([_f(vc), v.reshape(M, Hkv, 1, hd)], axis=2)
    o = np.zeros((M, qc))
    for m in range(M):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            p = special.softmax(K[m, g] @ q[m, h * hd:(h + 1) * hd] / np.sqrt(hd))
            o[m, h * hd:(h + 1) * hd] = p @ V[m, g]
    o = b(o)
    x1 = b(xf + (o @ _f(wo).T).astype(np.float32))
    n2 = b(x1 / np.sqrt(np.mean(x1 ** 2, 1, keepdims=True) + oracle.RMS_EPS) * _f(w_mlp))
    gu = (n2 @ _f(wgu).T).astype(np.float32).astype(np.float64)
    a = b(gu[:, :dff] * special.expit(gu[:, :dff]) * gu[:, dff:])
    xo = b(x1 + (a @ _f(wdown).T).astype(np.float32))
    for name, ref in (("n1", n1), ("qkv", qkv), ("o", o), ("x1", x1), ("n2", n2), ("a", a), ("x_out", xo)):
        got = _f(r[name])
        # each stage is compared on the previous stage's oracle value, so a
        # one-ulp rounding difference upstream may move a value by a few ulp
        assert np.all(np.abs(got - ref) <= 4 * oracle.bf16_ulp(ref) + 1e-30), name
        assert np.mean(got == ref) > 0.9, name
