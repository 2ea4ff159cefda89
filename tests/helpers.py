"""Shared pieces of the GPU tests: seeded inputs on the device and comparison
against the CPU oracle with the stated per-element tolerance."""
from __future__ import annotations

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
