"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.  It wraps ``oracle.c`` (plain C, double accumulation)
through ctypes; see that file for what each function computes and which
passage of the pages it restates.

Tolerance (stated with the method's target): a GPU fp32 output passes when
``|y_gpu - y| <= 2e-3 * sum_k |x w| + 1e-6``; a bf16 output gets one more bf16
ulp of the reference value.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

REL_TOL = 2e-3
ABS_TOL = 1e-6


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2, OpenMP); returns the .so path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
        lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, u16p, u16p,
                                    f64p, ctypes.c_void_p]
        lib.oracle_gemm.restype = None
        lib.oracle_bf16_from_float.argtypes = [ctypes.c_float]
        lib.oracle_bf16_from_float.restype = ctypes.c_uint16
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_num_threads.restype = ctypes.c_int
        f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
        lib.oracle_silu_gate.argtypes = [ctypes.c_long, f32p, f32p, u16p]
        lib.oracle_silu_gate.restype = None
        lib.oracle_layer.argtypes = [ctypes.c_int] * 4 + [u16p] * 5 + [ctypes.c_void_p] * 5
        lib.oracle_rmsnorm.argtypes = [ctypes.c_int, ctypes.c_int, u16p, u16p, ctypes.c_double, u16p]
        lib.oracle_rmsnorm.restype = None
        lib.oracle_gqa_decode.argtypes = [ctypes.c_int] * 5 + [u16p] * 5 + [u16p]
        lib.oracle_gqa_decode.restype = None
        lib.oracle_residual.argtypes = [ctypes.c_long, u16p, f64p, u16p]
        lib.oracle_residual.restype = None
        lib.oracle_layer.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def gemm(x_bits, w_bits, want_abs: bool = True):
    """Equation (1): y[m][n] = sum_k x[m][k] w[n][k] in double.

    x_bits: uint16 [M][K] (bf16), w_bits: uint16 [N][K] (bf16, K-major).
    Returns (y, absdot) as float64 [M][N]; absdot is None if not wanted.
    """
    x, w = _u16(x_bits), _u16(w_bits)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("K mismatch")
    y = np.empty((M, N), dtype=np.float64)
    a = np.empty((M, N), dtype=np.float64) if want_abs else None
    _load().oracle_gemm(M, K, N, x, w, y, a.ctypes.data if want_abs else None)
    return y, a


def bf16_from_f32(values) -> np.ndarray:
    """The oracle's own float -> bf16 RNE conversion, element by element."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32).ravel()
    out = np.fromiter((lib.oracle_bf16_from_float(float(f)) for f in v), dtype=np.uint16,
                      count=v.size)
    return out.reshape(np.shape(values))


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def silu(v: float) -> float:
    return float(_load().oracle_silu(float(v)))


def silu_gate(g, u) -> np.ndarray:
    """The chain's SiLU gate on fp32 gate and up values (same shape):
    bf16 bits of f32(silu(g) * u), silu in double."""
    g32 = np.ascontiguousarray(g, dtype=np.float32)
    u32 = np.ascontiguousarray(u, dtype=np.float32)
    if g32.shape != u32.shape:
        raise ValueError("shape mismatch")
    out = np.empty(g32.shape, dtype=np.uint16)
    _load().oracle_silu_gate(g32.size, g32.ravel(), u32.ravel(), out.reshape(-1))
    return out


def layer(x_bits, wq, wo, wgu, wdown):
    """One chain layer; returns dict of h1, h2, a, x_out (bf16 bits) and y_f32."""
    x = _u16(x_bits)
    wq, wo, wgu, wdown = _u16(wq), _u16(wo), _u16(wgu), _u16(wdown)
    M, d = x.shape
    q = wq.shape[0]
    dff = wgu.shape[0] // 2
    assert wq.shape == (q, d) and wo.shape == (d, q)
    assert wgu.shape == (2 * dff, d) and wdown.shape == (d, dff)
    h1 = np.empty((M, q), np.uint16)
    h2 = np.empty((M, d), np.uint16)
    a = np.empty((M, dff), np.uint16)
    xo = np.empty((M, d), np.uint16)
    y = np.empty((M, d), np.float32)
    _load().oracle_layer(M, d, q, dff, x, wq, wo, wgu, wdown, h1.ctypes.data, h2.ctypes.data,
                         a.ctypes.data, xo.ctypes.data, y.ctypes.data)
    return {"h1": h1, "h2": h2, "a": a, "x_out": xo, "y_f32": y}


def chain(x0_bits, layers):
    """Run the chain over ``layers`` = iterable of (wq, wo, wgu, wdown)."""
    x = _u16(x0_bits)
    outs = []
    for (wq, wo, wgu, wdown) in layers:
        r = layer(x, wq, wo, wgu, wdown)
        outs.append(r)
        x = r["x_out"]
    return outs


def bound(absdot, y_ref=None, bf16_out: bool = False) -> np.ndarray:
    """Per-element tolerance: 2e-3 * sum|x w| + 1e-6 (+ 1 bf16 ulp of y_ref)."""
    b = REL_TOL * np.asarray(absdot, dtype=np.float64) + ABS_TOL
    if bf16_out:
        b = b + bf16_ulp(y_ref)
    return b


def bf16_ulp(v) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (2**(e-7) for normal v, 2**-133 below)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(v > 0, np.exp2(e - 7.0), 2.0 ** -133)


def timed_gemm(x_bits, w_bits):
    """(seconds, threads) of one oracle_gemm call, for the CPU baseline."""
    t0 = time.perf_counter()
    gemm(x_bits, w_bits, want_abs=False)
    return time.perf_counter() - t0, num_threads()


RMS_EPS = 1e-6   # the RMSNorm epsilon of the decoder layer


def rmsnorm(x_bits, w_bits, eps: float = RMS_EPS) -> np.ndarray:
    """bf16(x / sqrt(mean(x^2) + eps) * w) per row of x [M][d], in double."""
    x, w = _u16(x_bits), _u16(w_bits)
    M, d = x.shape
    if w.shape != (d,):
        raise ValueError("weight shape")
    out = np.empty((M, d), np.uint16)
    _load().oracle_rmsnorm(M, d, x, w, float(eps), out)
    return out


def gqa_decode(q_bits, kc_bits, vc_bits, kn_bits, vn_bits, Hq: int, Hkv: int) -> np.ndarray:
    """Grouped-query decode attention (see oracle.c): q [M][Hq*hd], caches
    [M][Hkv][T][hd], new key/value [M][Hkv*hd]; returns bf16 bits [M][Hq*hd]."""
    q, kc, vc = _u16(q_bits), _u16(kc_bits), _u16(vc_bits)
    kn, vn = _u16(kn_bits), _u16(vn_bits)
    M, Hkv_, T, hd = kc.shape
    if Hkv_ != Hkv or q.shape != (M, Hq * hd) or vc.shape != kc.shape or kn.shape != (M, Hkv * hd) \
            or vn.shape != kn.shape or Hq % Hkv:
        raise ValueError("attention shapes")
    out = np.empty((M, Hq * hd), np.uint16)
    _load().oracle_gqa_decode(M, Hq, Hkv, hd, T, q, kc.reshape(-1), vc.reshape(-1), kn, vn, out)
    return out


def residual(x_bits, y) -> np.ndarray:
    """bf16(f32(x + f32(y))) elementwise: x bf16 bits, y the projection's double result."""
    x = _u16(x_bits)
    yy = np.ascontiguousarray(y, dtype=np.float64)
    if yy.shape != x.shape:
        raise ValueError("shape mismatch")
    out = np.empty(x.shape, np.uint16)
    _load().oracle_residual(x.size, x.reshape(-1), yy.reshape(-1), out.reshape(-1))
    return out


def decoder_layer(x_bits, w_attn, wqkv, kc, vc, wo, w_mlp, wgu, wdown, Hq: int, Hkv: int,
                  eps: float = RMS_EPS):
    """One decoder layer (see oracle.c): returns dict of n1, qkv, o, x1, n2, a, x_out (bf16 bits)
    and the pieces of qkv (q, k, v)."""
    x = _u16(x_bits)
    M, d = x.shape
    hd = kc.shape[3]
    qc, kvc = Hq * hd, Hkv * hd
    n1 = rmsnorm(x, w_attn, eps)
    y, _ = gemm(n1, wqkv, want_abs=False)
    qkv = _bf16_of_f64(y)
    q, k, v = qkv[:, :qc], qkv[:, qc:qc + kvc], qkv[:, qc + kvc:qc + 2 * kvc]
    o = gqa_decode(q, kc, vc, k, v, Hq, Hkv)
    yo, _ = gemm(o, wo, want_abs=False)
    x1 = residual(x, yo)
    n2 = rmsnorm(x1, w_mlp, eps)
    ygu, _ = gemm(n2, wgu, want_abs=False)
    dff = wgu.shape[0] // 2
    a = silu_gate(ygu[:, :dff].astype(np.float32), ygu[:, dff:].astype(np.float32))
    yd, _ = gemm(a, wdown, want_abs=False)
    x_out = residual(x1, yd)
    return {"n1": n1, "qkv": qkv, "q": q, "k": k, "v": v, "o": o, "x1": x1, "n2": n2, "a": a, "x_out": x_out}


def _bf16_of_f64(y) -> np.ndarray:
    """bf16 bits of f32(y) for a large array, by the oracle's own rounding rule
    applied through residual() with a zero residual (bf16(f32(0 + f32(y))))."""
    zero = np.zeros(np.shape(y), np.uint16)
    return residual(zero, y)
