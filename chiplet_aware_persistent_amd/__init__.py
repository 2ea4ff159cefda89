"""Python binding of libsgemm.so: the small-M decode GEMM and the persistent
layer chain for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  The functions mirror the C ABI of include/sgemm.h
(same names, same arguments, device pointers as integers); ``Gemm`` and
``LayerChain`` are conveniences that take torch tensors and streams.  PyTorch
is used only to own device memory and streams.

If the library has not been built (``python -m chiplet_aware_persistent_amd.build``)
importing works but every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgemm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "sgemm.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_TIMEOUT, ERR_WORKSPACE, ERR_TOPOLOGY = 0, -1, -2, -3, -4, -5, -6
KIND_GEMM, KIND_LAYERCHAIN, KIND_DECODER = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1
F_FORCE_DOT2 = 1 << 0
F_FORCE_MFMA = 1 << 1
F_W_CACHED = 1 << 2
F_SYNC_FLAT = 1 << 3
F_SYNC_AGENT = 1 << 4
F_STAMPS = 1 << 5
F_WATCHDOG_TEST = 1 << 6
F_W_SC1 = 1 << 7
F_POLL_LEADER = 1 << 8
F_MTILE_ITEMS = 1 << 9
F_LAUNCH_PER_STAGE = 1 << 10
F_SCHEDULER = 1 << 11
F_CHECK_PLACEMENT = 1 << 12
F_KCHUNK = 1 << 13
F_MSPLIT = 1 << 14


class SgemmError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__("%s: %s (%d)" % (what or "sgemm", status_string(code), code))


class Problem(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("M", ctypes.c_int), ("K", ctypes.c_int), ("N", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("n_layers", ctypes.c_int), ("d_model", ctypes.c_int),
                ("q_cols", ctypes.c_int), ("d_ff", ctypes.c_int), ("flags", ctypes.c_uint),
                ("tn", ctypes.c_int), ("splitk", ctypes.c_int), ("waves", ctypes.c_int),
                ("kslices", ctypes.c_int), ("tm", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ctx", ctypes.c_int)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libsgemm.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsgemm.so is not built; run `python -m chiplet_aware_persistent_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.sgemm_plan_create.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, ctypes.POINTER(vp),
                                          ctypes.POINTER(sz)]
        lib.sgemm_plan_destroy.argtypes = [vp]
        lib.sgemm_workspace_init.argtypes = [vp, vp, vp]
        lib.sgemm_run.argtypes = [vp, vp, vp, vp, vp, vp]
        lib.layerchain_run.argtypes = [vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                       ctypes.POINTER(vp), vp, vp, vp, vp]
        lib.sgemm_chain_buffer.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz),
                                           ctypes.POINTER(sz)]
        lib.sgemm_query_status.argtypes = [vp, vp, vp]
        lib.sgemm_status_string.argtypes = [ctypes.c_int]
        lib.sgemm_status_string.restype = ctypes.c_char_p
        lib.sgemm_plan_describe.argtypes = [vp, ctypes.c_char_p, sz]
        lib.sgemm_topology_probe.argtypes = [vp, ctypes.c_int, vp]
        lib.sgemm_read_probe.argtypes = [vp, sz, ctypes.c_int, vp, ctypes.c_int, vp]
        lib.sgemm_device_check.argtypes = [ctypes.c_int]
        lib.sgemm_run_noalloc.argtypes = [vp, vp, vp, vp, vp]
        lib.decoder_run.argtypes = [vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp]
        for f in ("sgemm_plan_create", "sgemm_plan_destroy", "sgemm_workspace_init", "sgemm_run",
                  "layerchain_run", "sgemm_chain_buffer", "sgemm_query_status", "sgemm_plan_describe",
                  "sgemm_topology_probe", "sgemm_read_probe", "sgemm_device_check", "sgemm_run_noalloc", "decoder_run"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/sgemm.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|const char\*)\s+(\w+)\s*\(", text)))


# ------------------------------------------------------------ C-ABI mirrors
def status_string(code: int) -> str:
    try:
        return library().sgemm_status_string(int(code)).decode()
    except RuntimeError:
        return "status %d" % code


def sgemm_plan_create(problem: Problem, device: int = 0):
    """Returns (status, plan handle, workspace bytes)."""
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    rc = library().sgemm_plan_create(ctypes.byref(problem), int(device), ctypes.byref(h), ctypes.byref(ws))
    return rc, h.value, ws.value


def sgemm_plan_destroy(plan) -> int:
    return library().sgemm_plan_destroy(plan)


def sgemm_workspace_init(plan, workspace: int, stream: int = 0) -> int:
    return library().sgemm_workspace_init(plan, workspace, stream)


def sgemm_run(plan, X: int, W: int, Y: int, workspace: int, stream: int = 0) -> int:
    return library().sgemm_run(plan, X, W, Y, workspace, stream)


def sgemm_run_noalloc(plan, X: int, W: int, Y: int, stream: int = 0) -> int:
    return library().sgemm_run_noalloc(plan, X, W, Y, stream)


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*[int(p) for p in ptrs])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr


def layerchain_run(plan, X0: int, Wq, Wo, Wgu, Wdown, Y_f32: int, Y_bf16: int, workspace: int,
                   stream: int = 0) -> int:
    a = [_ptr_array(p) for p in (Wq, Wo, Wgu, Wdown)]
    return library().layerchain_run(plan, X0, a[0][0], a[1][0], a[2][0], a[3][0], Y_f32, Y_bf16 or None,
                                    workspace, stream)


def decoder_run(plan, X0: int, w_norm: int, Wqkv, Wo, Wgu, Wdown, K_cache: int, V_cache: int, Y_f32: int,
                Y_bf16: int, workspace: int, stream: int = 0) -> int:
    a = [_ptr_array(p) for p in (Wqkv, Wo, Wgu, Wdown)]
    return library().decoder_run(plan, X0, w_norm, a[0][0], a[1][0], a[2][0], a[3][0], K_cache or None,
                                 V_cache or None, Y_f32, Y_bf16 or None, workspace, stream)


def sgemm_chain_buffer(plan, layer: int, which: int):
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    rc = library().sgemm_chain_buffer(plan, layer, which, ctypes.byref(off), ctypes.byref(nb))
    return rc, off.value, nb.value


def sgemm_query_status(plan, workspace: int, stream: int = 0) -> int:
    return library().sgemm_query_status(plan, workspace, stream)


def sgemm_plan_describe(plan) -> dict:
    n = library().sgemm_plan_describe(plan, None, 0)
    buf = ctypes.create_string_buffer(max(n, 1))
    library().sgemm_plan_describe(plan, buf, n)
    return json.loads(buf.value.decode())


def sgemm_device_check(device: int = 0) -> int:
    return library().sgemm_device_check(int(device))


def sgemm_topology_probe(xcc_out: int, n_wg: int, stream: int = 0) -> int:
    return library().sgemm_topology_probe(xcc_out, n_wg, stream)


def sgemm_read_probe(src: int, nbytes: int, pattern: int, sink: int, grid: int = 256, stream: int = 0) -> int:
    return library().sgemm_read_probe(src, nbytes, pattern, sink, grid, stream)


# ------------------------------------------------------------ conveniences
def _stream_handle(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, what: str):
    if rc != OK:
        raise SgemmError(rc, what)


def _need(t, shape, dtype, name):
    """Raise ValueError unless tensor t has this shape and dtype and is contiguous."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise ValueError("%s: expected dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)


def _need_workspace(ws, nbytes):
    import torch

    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace: expected a contiguous 1-D uint8 tensor")
    if ws.numel() < nbytes:
        raise ValueError("workspace: %d bytes, the plan needs %d" % (ws.numel(), nbytes))


class _PlanBase:
    def __init__(self, problem: Problem, device: int):
        rc, h, ws = sgemm_plan_create(problem, device)
        _check(rc, "sgemm_plan_create")
        self.handle, self.workspace_bytes, self.device = h, ws, device
        self.problem = problem

    def describe(self) -> dict:
        return sgemm_plan_describe(self.handle)

    def new_workspace(self, stream=None):
        import torch

        ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device="cuda:%d" % self.device)
        _check(sgemm_workspace_init(self.handle, ws.data_ptr(), _stream_handle(stream)), "sgemm_workspace_init")
        return ws

    def status(self, workspace, stream=None) -> int:
        return sgemm_query_status(self.handle, workspace.data_ptr(), _stream_handle(stream))

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.sgemm_plan_destroy(h)
            self.handle = None


class Gemm(_PlanBase):
    """Y[M,N] = X[M,K] . W^T with W stored [N][K] (K-major), bf16 in, fp32 (or bf16) out."""

    def __init__(self, M: int, K: int, N: int, out_dtype: int = OUT_F32, flags: int = 0, tn: int = 0,
                 splitk: int = 0, waves: int = 0, kslices: int = 0, device: int = 0, tm: int = 0):
        p = Problem(KIND_GEMM, M, K, N, out_dtype, 0, 0, 0, 0, flags, tn, splitk, waves, kslices, tm)
        super().__init__(p, device)
        self.M, self.K, self.N, self.out_dtype = M, K, N, out_dtype

    def __call__(self, X, W, Y, workspace, stream=None):
        import torch

        _need(X, (self.M, self.K), torch.bfloat16, "X")
        _need(W, (self.N, self.K), torch.bfloat16, "W")
        _need(Y, (self.M, self.N), torch.float32 if self.out_dtype == OUT_F32 else torch.bfloat16, "Y")
        _need_workspace(workspace, self.workspace_bytes)
        _check(sgemm_run(self.handle, X.data_ptr(), W.data_ptr(), Y.data_ptr(), workspace.data_ptr(),
                         _stream_handle(stream)), "sgemm_run")
        return Y


class LayerChain(_PlanBase):
    """The per-layer projection chain (Q, O, gate_up + SiLU gate, down) in one launch."""

    def __init__(self, M: int, n_layers: int, d_model: int, q_cols: int, d_ff: int, flags: int = 0,
                 tn: int = 0, splitk: int = 0, waves: int = 0, kslices: int = 0, device: int = 0):
        p = Problem(KIND_LAYERCHAIN, M, 0, 0, 0, n_layers, d_model, q_cols, d_ff, flags, tn, splitk, waves,
                    kslices)
        super().__init__(p, device)
        self.M, self.n_layers, self.d, self.q, self.dff = M, n_layers, d_model, q_cols, d_ff

    def __call__(self, X0, Wq, Wo, Wgu, Wdown, Y_f32, workspace, Y_bf16=None, stream=None):
        import torch

        L = self.n_layers
        if not (len(Wq) == len(Wo) == len(Wgu) == len(Wdown) == L):
            raise ValueError("expected %d weight tensors per projection" % L)
        for l in range(L):
            _need(Wq[l], (self.q, self.d), torch.bfloat16, "Wq[%d]" % l)
            _need(Wo[l], (self.d, self.q), torch.bfloat16, "Wo[%d]" % l)
            _need(Wgu[l], (2 * self.dff, self.d), torch.bfloat16, "Wgu[%d]" % l)
            _need(Wdown[l], (self.d, self.dff), torch.bfloat16, "Wdown[%d]" % l)
        _need(X0, (self.M, self.d), torch.bfloat16, "X0")
        _need(Y_f32, (self.M, self.d), torch.float32, "Y_f32")
        if Y_bf16 is not None:
            _need(Y_bf16, (self.M, self.d), torch.bfloat16, "Y_bf16")
        _need_workspace(workspace, self.workspace_bytes)
        _check(layerchain_run(self.handle, X0.data_ptr(), [w.data_ptr() for w in Wq],
                              [w.data_ptr() for w in Wo], [w.data_ptr() for w in Wgu],
                              [w.data_ptr() for w in Wdown], Y_f32.data_ptr(),
                              Y_bf16.data_ptr() if Y_bf16 is not None else 0, workspace.data_ptr(),
                              _stream_handle(stream)), "layerchain_run")
        return Y_f32

    def activation(self, workspace, layer: int, which: int):
        """View of an intermediate activation kept in the workspace (bf16 [M][cols])."""
        import torch

        rc, off, nb = sgemm_chain_buffer(self.handle, layer, which)
        _check(rc, "sgemm_chain_buffer")
        cols = nb // (2 * self.M)
        return workspace[off:off + nb].view(torch.bfloat16).view(self.M, cols)


def read_probe(buf, pattern: int = 0, sink=None, grid: int = 256, nbytes: int | None = None):
    """Enqueue one streaming read of ``buf`` (a CUDA tensor) on the current stream;
    xors its 32-bit words into ``sink`` (an int32 CUDA tensor of one element,
    created zeroed when None) and returns ``sink``."""
    import torch

    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(sgemm_read_probe(buf.data_ptr(), n, pattern, sink.data_ptr(), grid, _stream_handle(None)),
           "sgemm_read_probe")
    return sink


def topology(n_wg: int = 256, device: int = 0):
    """XCC id of each of n_wg workgroups of one launch (list of ints)."""
    import torch

    out = torch.full((n_wg,), -1, dtype=torch.int32, device="cuda:%d" % device)
    _check(sgemm_topology_probe(out.data_ptr(), n_wg, _stream_handle(None)), "sgemm_topology_probe")
    torch.cuda.synchronize()
    return out.cpu().tolist()


class Decoder(_PlanBase):
    """The whole decoder layer (RMSNorm, QKV, grouped-query decode attention,
    O with residual, RMSNorm, gate_up with SiLU gate, down with residual), all
    layers in one persistent launch."""

    def __init__(self, M: int, n_layers: int, d_model: int, d_ff: int, n_heads: int, n_kv_heads: int,
                 head_dim: int, ctx: int, flags: int = 0, tn: int = 0, splitk: int = 0, waves: int = 0,
                 kslices: int = 0, device: int = 0):
        p = Problem(KIND_DECODER, M, 0, 0, 0, n_layers, d_model, 0, d_ff, flags, tn, splitk, waves, kslices, 0,
                    n_heads, n_kv_heads, head_dim, ctx)
        super().__init__(p, device)
        self.M, self.n_layers, self.d, self.dff = M, n_layers, d_model, d_ff
        self.Hq, self.Hkv, self.hd, self.T = n_heads, n_kv_heads, head_dim, ctx
        self.q, self.kv = n_heads * head_dim, n_kv_heads * head_dim

    def __call__(self, X0, w_norm, Wqkv, Wo, Wgu, Wdown, K_cache, V_cache, Y_f32, workspace, Y_bf16=None,
                 stream=None):
        import torch

        L = self.n_layers
        if not (len(Wqkv) == len(Wo) == len(Wgu) == len(Wdown) == L):
            raise ValueError("expected %d weight tensors per projection" % L)
        for l in range(L):
            _need(Wqkv[l], (self.q + 2 * self.kv, self.d), torch.bfloat16, "Wqkv[%d]" % l)
            _need(Wo[l], (self.d, self.q), torch.bfloat16, "Wo[%d]" % l)
            _need(Wgu[l], (2 * self.dff, self.d), torch.bfloat16, "Wgu[%d]" % l)
            _need(Wdown[l], (self.d, self.dff), torch.bfloat16, "Wdown[%d]" % l)
        _need(X0, (self.M, self.d), torch.bfloat16, "X0")
        _need(w_norm, (L, 2, self.d), torch.bfloat16, "w_norm")
        cache = (L, self.M, self.Hkv, self.T, self.hd)
        _need(K_cache, cache, torch.bfloat16, "K_cache")
        _need(V_cache, cache, torch.bfloat16, "V_cache")
        _need(Y_f32, (self.M, self.d), torch.float32, "Y_f32")
        if Y_bf16 is not None:
            _need(Y_bf16, (self.M, self.d), torch.bfloat16, "Y_bf16")
        _need_workspace(workspace, self.workspace_bytes)
        _check(decoder_run(self.handle, X0.data_ptr(), w_norm.data_ptr(), [w.data_ptr() for w in Wqkv],
                           [w.data_ptr() for w in Wo], [w.data_ptr() for w in Wgu], [w.data_ptr() for w in Wdown],
                           K_cache.data_ptr() if self.T else 0, V_cache.data_ptr() if self.T else 0,
                           Y_f32.data_ptr(), Y_bf16.data_ptr() if Y_bf16 is not None else 0, workspace.data_ptr(),
                           _stream_handle(stream)), "decoder_run")
        return Y_f32

    def activation(self, workspace, layer: int, which: int):
        """View of an intermediate kept in the workspace: which = 0 qkv, 1 o,
        2 x1, 3 a, 4 x' (bf16 [M][cols])."""
        import torch

        rc, off, nb = sgemm_chain_buffer(self.handle, layer, which)
        _check(rc, "sgemm_chain_buffer")
        cols = nb // (2 * self.M)
        return workspace[off:off + nb].view(torch.bfloat16).view(self.M, cols)
