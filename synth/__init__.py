"""Seeded synthetic inputs for the small-M decode GEMM and the layer chain.

This module only draws numbers; it holds none of the GEMM arithmetic.  The
tests, the bench and the golden-value scripts take their inputs from here and
hand the very same bf16 bit patterns to the HIP library and to the oracle.

Generator
---------
SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), used counter-style:

* ``key(seed)``   = the first output of SplitMix64 started from state ``seed``;
* element ``i``   = the ``(i+1)``-th output of SplitMix64 started from ``key``,
  i.e. ``mix(key + (i+1)*GAMMA)``, so any slice of a tensor can be drawn
  without drawing what precedes it.

Element ``i`` of a ``[rows][cols]`` tensor is its row-major linear index.

Distributions
-------------
* uniform in [0,1): ``u = (r >> 11) * 2**-53`` (exact in double);
* U(-a, a): ``(2u - 1) * a`` in double, rounded to fp32 (RNE) and then to bf16
  (RNE).  Only IEEE-exact or correctly rounded operations are used, so the
  numpy side and the torch side below give identical bits on any device;
* N(0, 1): Box-Muller on elements ``2i`` and ``2i+1``:
  ``sqrt(-2 ln(1 - u0)) * cos(2 pi u1)`` in double, then fp32, then bf16.
  Host only (it calls libm), which is fine: activations are small.
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Tensor ids used in seeds.
T_X, T_WQ, T_WO, T_WGU, T_WDOWN = 0, 1, 2, 3, 4


def seed_for(workload: int, layer: int = 0, tensor: int = 0, variant: int = 0) -> int:
    """Seed scheme: one 64-bit seed per (workload, layer, tensor, variant).
    Workloads: 1 the 1x1024x1024 GEMM, 2 the decode projections at M = 1,
    3 the same shapes at M = 8..64, 4 the K = 7168 GEMMs, 5 the 36-layer chain."""
    return (0x5EED0000 + (workload << 16) + (layer << 8) + (tensor << 4) + variant) & MASK64


# ---------------------------------------------------------------- reference
def _mix_py(z: int) -> int:
    z = ((z ^ (z >> 30)) * MUL1) & MASK64
    z = ((z ^ (z >> 27)) * MUL2) & MASK64
    return z ^ (z >> 31)


def splitmix64_sequence(state: int, count: int) -> list[int]:
    """Plain sequential SplitMix64 (pure Python), for pinning the vectorised one."""
    out = []
    for _ in range(count):
        state = (state + GAMMA) & MASK64
        out.append(_mix_py(state))
    return out


def key(seed: int) -> int:
    return splitmix64_sequence(seed & MASK64, 1)[0]


# ---------------------------------------------------------------- numpy side
def _mix_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
    return z ^ (z >> np.uint64(31))


def stream_u64(seed: int, start: int, count: int) -> np.ndarray:
    """Elements start .. start+count-1 of the counter stream of ``seed``."""
    k = np.uint64(key(seed))
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix_np(k + idx * np.uint64(GAMMA))


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    r = stream_u64(seed, start, count)
    return (r >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even; NaN stays NaN."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    q = ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return np.where(nan, q, r)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform_bf16(seed: int, rows: int, cols: int, a: float, row_start: int = 0) -> np.ndarray:
    """bf16 bits [rows][cols] of U(-a, a); rows row_start .. row_start+rows-1."""
    u = uniform01(seed, row_start * cols, rows * cols)
    v = ((2.0 * u - 1.0) * a).astype(np.float32)
    return f32_to_bf16_bits(v).reshape(rows, cols)


def uniform_bf16_rows(seed: int, cols: int, a: float, row_ids) -> np.ndarray:
    """Arbitrary (sampled) rows of the same tensor as ``uniform_bf16``."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    out = np.empty((len(row_ids), cols), dtype=np.uint16)
    for i, r in enumerate(row_ids):
        out[i] = uniform_bf16(seed, 1, cols, a, row_start=int(r))[0]
    return out


def normal_bf16(seed: int, rows: int, cols: int) -> np.ndarray:
    n = rows * cols
    u = uniform01(seed, 0, 2 * n)
    u0, u1 = u[0::2], u[1::2]
    z = np.sqrt(-2.0 * np.log1p(-u0)) * np.cos(2.0 * math.pi * u1)
    return f32_to_bf16_bits(z.astype(np.float32)).reshape(rows, cols)


def int_bf16(seed: int, rows: int, cols: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi] (exact in bf16 for |v| <= 256)."""
    r = stream_u64(seed, 0, rows * cols)
    v = (r % np.uint64(hi - lo + 1)).astype(np.int64) + lo
    return f32_to_bf16_bits(v.astype(np.float32)).reshape(rows, cols)


def weight_scale(K: int) -> float:
    """a = 1/sqrt(K) of U(-a, a), computed once on the host (correctly rounded)."""
    return 1.0 / math.sqrt(K)


# ---------------------------------------------------------------- torch side
def uniform_bf16_torch(seed: int, rows: int, cols: int, a: float, device, out=None,
                       chunk_elems: int = 1 << 25):
    """Same bits as ``uniform_bf16`` drawn with torch int64 ops on ``device``.

    int64 arithmetic wraps modulo 2**64 in torch on every backend; logical
    shifts are emulated by masking the arithmetic ones.
    """
    import torch

    def s64(v: int) -> int:
        v &= MASK64
        return v - (1 << 64) if v >= (1 << 63) else v

    def lsr(z, s):
        return (z >> s) & ((1 << (64 - s)) - 1)

    n = rows * cols
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    k = s64(key(seed))
    g, m1, m2 = s64(GAMMA), s64(MUL1), s64(MUL2)
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        z = torch.arange(s + 1, e + 1, dtype=torch.int64, device=device)
        z = z * g + k
        z = (z ^ lsr(z, 30)) * m1
        z = (z ^ lsr(z, 27)) * m2
        z = z ^ lsr(z, 31)
        u = lsr(z, 11).to(torch.float64) * (2.0 ** -53)
        flat[s:e] = ((2.0 * u - 1.0) * a).to(torch.float32).to(torch.bfloat16)
        del z, u
    return out


def to_torch_bf16(bits: np.ndarray, device="cpu"):
    """Host bf16 bit array -> torch.bfloat16 tensor (bit copy)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_torch_bf16(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
