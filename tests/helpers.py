"""Shared pieces of the GPU tests: seeded inputs on the device and comparison
against the CPU oracle with the stated per-element tolerance."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import synth


def device_tensor_bf16(bits: np.ndarray, dev):
    return synth.to_torch_bf16(bits, dev)


def host_bits(t) -> np.ndarray:
    return synth.from_torch_bf16(t)


def gemm_inputs(M: int, K: int, N: int, seed_x: int, seed_w: int, dev, w_on_device: bool = False):
    """X ~ N(0,1) and W ~ U(-1/sqrt(K), 1/sqrt(K)), bf16 bits.

    Returns (x_bits, w_bits or None, X, W).  With w_on_device the weights are
    drawn on the GPU (same bits as the host generator) and w_bits is None;
    use sampled_w_rows() for the oracle then.
    """
    import torch

    x_bits = synth.normal_bf16(seed_x, M, K)
    X = device_tensor_bf16(x_bits, dev)
    a = synth.weight_scale(K)
    if w_on_device:
        W = synth.uniform_bf16_torch(seed_w, N, K, a, dev)
        return x_bits, None, X, W
    w_bits = synth.uniform_bf16(seed_w, N, K, a)
    return x_bits, w_bits, X, device_tensor_bf16(w_bits, dev)


def report(case: str, ratio: float, **extra):
    """Print a parity figure (max |delta| / bound) and, when the environment
    names a file in SGEMM_PARITY_REPORT, append it there as one JSON line."""
    print("parity %s: max |delta|/bound = %.4g" % (case, ratio), flush=True)
    path = os.environ.get("SGEMM_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(case=case, max_ratio=ratio, **extra)) + "\n")


def device_weights_checked(W, seed_w: int, K: int, rows=None) -> np.ndarray:
    """Host copy of weights drawn on the device by the counter-based
    generator, after checking a few whole rows against the host generator."""
    w = host_bits(W)
    N = w.shape[0]
    rows = sorted({0, N // 2, N - 1} if rows is None else set(rows))
    import synth

    ref = synth.uniform_bf16_rows(seed_w, K, synth.weight_scale(K), np.array(rows, dtype=np.int64))
    assert np.array_equal(w[rows], ref)
    return w


def sampled_columns(N: int, count: int, seed: int = 0) -> np.ndarray:
    """Columns to check at full size: both ends of every XCD block plus random ones."""
    rng = np.random.default_rng(seed)
    nx = -(-N // 8)
    ends = set()
    for x in range(8):
        for c in (x * nx, x * nx + 1, x * nx + nx - 1, x * nx + nx // 2):
            if 0 <= c < N:
                ends.add(c)
    ends.update(rng.choice(N, size=min(count, N), replace=False).tolist())
    ends.add(N - 1)
    return np.array(sorted(ends), dtype=np.int64)


def check(y_gpu: np.ndarray, x_bits: np.ndarray, w_rows_bits: np.ndarray, bf16_out: bool = False):
    """Compare GPU outputs (float array [M][len(cols)]) with the oracle on the
    given weight rows.  Returns max |delta| / bound; asserts it is <= 1."""
    y_ref, absdot = oracle.gemm(x_bits, w_rows_bits)
    bound = oracle.bound(absdot, y_ref=y_ref, bf16_out=bf16_out)
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    if ratio > 1.0:
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError("parity violated at %s: gpu=%r ref=%r bound=%r (ratio %.3g)"
                             % (i, float(y_gpu[i]), float(y_ref[i]), float(bound[i]), ratio))
    return ratio


# Forced-plan parity cases.  Each list holds combinations the planner accepts
# (the GPU parity tests run them); the *_REFUSED lists hold combinations it
# refuses with SGEMM_ERR_UNSUPPORTED because the X window of the forced split or
# the K-slice buffers do not fit the LDS, or a slice would be empty (a CPU test
# checks the refusal).
KSL_SHAPES = [(16, 4096, 1040), (33, 2056, 777), (64, 1000, 530), (20, 12288, 300), (48, 520, 64)]
KSL_REFUSED = [(33, 2056, 777, 8, 0), (33, 2056, 777, 8, 3), (64, 1000, 530, 4, 3), (64, 1000, 530, 8, 3),
               (20, 12288, 300, 2, 3), (20, 12288, 300, 4, 3), (20, 12288, 300, 8, 3), (48, 520, 64, 4, 0),
               (48, 520, 64, 4, 3), (48, 520, 64, 8, 0), (48, 520, 64, 8, 3)]
KSL_CASES = [(M, K, N, ksl, s) for (M, K, N) in KSL_SHAPES for ksl in (2, 4, 8) for s in (0, 3)
             if (M, K, N, ksl, s) not in KSL_REFUSED]
MTI_SHAPES = [(17, 776, 530), (33, 2056, 900), (64, 4096, 1536), (48, 520, 64), (64, 12288, 4096)]
MTI_REFUSED = [(64, 4096, 1536, 3), (64, 12288, 4096, 3)]
MTI_CASES = [(M, K, N, s) for (M, K, N) in MTI_SHAPES for s in (0, 3) if (M, K, N, s) not in MTI_REFUSED]
SPLITK_SHAPES = [(1, 1024, 1024), (4, 2056, 999), (8, 4096, 512), (12, 776, 530), (16, 1024, 2048),
                 (33, 2048, 1536), (64, 1000, 1000)]
