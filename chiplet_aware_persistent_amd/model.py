"""Closed-form performance model used for reporting (not part of the compute path).

* Eq.(1) of the Fleet reading note (section 3f, "L2 hit rate model"): with R =
  min(W, m_tiles) workers sharing a weight column, the weight L2 hit rate is
  (R - 1) / R, m_tiles = ceil(B / T_M).
* Effective arithmetic intensity (same section, auxiliary equation / Figure 7):
  AI_eff = B / (1 - hit).
* Roofline floor of a decode GEMM on MI355X: weight bytes 2*K*N over the HBM peak.
"""
from __future__ import annotations

import math

HBM_PEAK_BPS = 8.0e12          # MI355X HBM3E peak
BF16_MFMA_PEAK = 2.5e15        # dense bf16 MFMA, FLOP/s


def eq1_hit(B: int, W: int = 32, T_M: int = 16) -> float:
    """Predicted weight L2 hit rate of M-major windowed traversal, Eq.(1)."""
    m_tiles = math.ceil(B / T_M)
    R = min(W, m_tiles)
    return (R - 1) / R


def ai_eff(B: float, hit: float) -> float:
    """FLOP per HBM byte after L2 reuse: B / (1 - hit)."""
    return B / (1.0 - hit)


def weight_bytes(K: int, N: int) -> int:
    return 2 * K * N


def algorithmic_bytes(M: int, K: int, N: int, out_bytes: int = 4) -> int:
    """Bytes a decode GEMM must move: W once, X once, Y once."""
    return 2 * K * N + 2 * M * K + out_bytes * M * N


def floor_us(K: int, N: int, peak: float = HBM_PEAK_BPS) -> float:
    return weight_bytes(K, N) / peak * 1e6


def ridge_flop_per_byte() -> float:
    return BF16_MFMA_PEAK / HBM_PEAK_BPS
