"""CPU-side checks of the C ABI and the host logic: the library loads, exports
every function the header declares, rejects bad arguments before enqueuing
anything, and the planner's decompositions cover every output column and K
value exactly once.  No GPU is needed (plan creation does not touch HIP)."""
import json
import math
import os

import numpy as np
import pytest

import chiplet_aware_persistent_amd as sg
from chiplet_aware_persistent_amd import model

GOLD = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(sg.LIB_PATH), reason="libsgemm.so not built")


def test_exports_every_header_function():
    names = sg.header_functions()
    assert len(names) >= 10
    lib = sg.library()
    for n in names:
        assert hasattr(lib, n), n


def _create(**kw):
    p = sg.Problem(kw.get("kind", sg.KIND_GEMM), kw.get("M", 1), kw.get("K", 64), kw.get("N", 64),
                   kw.get("out", sg.OUT_F32), kw.get("L", 0), kw.get("d", 0), kw.get("q", 0), kw.get("dff", 0),
                   kw.get("flags", 0), kw.get("tn", 0), kw.get("splitk", 0), kw.get("waves", 0),
                   kw.get("ksl", 0), kw.get("tm", 0))
    rc, h, ws = sg.sgemm_plan_create(p)
    if h:
        sg.sgemm_plan_destroy(h)
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), sg.ERR_INVALID_ARG),
    (dict(M=257), sg.ERR_UNSUPPORTED),
    (dict(K=12), sg.ERR_INVALID_ARG),
    (dict(K=0), sg.ERR_INVALID_ARG),
    (dict(N=0), sg.ERR_INVALID_ARG),
    (dict(out=7), sg.ERR_INVALID_ARG),
    (dict(flags=sg.F_FORCE_DOT2 | sg.F_FORCE_MFMA), sg.ERR_INVALID_ARG),
    (dict(waves=3), sg.ERR_INVALID_ARG),
    (dict(splitk=65), sg.ERR_UNSUPPORTED),
    (dict(ksl=3), sg.ERR_INVALID_ARG),
    (dict(ksl=-1), sg.ERR_INVALID_ARG),
    (dict(M=4, ksl=2), sg.ERR_UNSUPPORTED),               # K slices are an MFMA-path option
    (dict(M=16, K=4096, N=4096, ksl=8), sg.OK),
    (dict(kind=9), sg.ERR_INVALID_ARG),
    (dict(K=1 << 20, N=1 << 12), sg.ERR_UNSUPPORTED),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=0, d=64, q=64, dff=64), sg.ERR_INVALID_ARG),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=2, d=60, q=64, dff=64), sg.ERR_INVALID_ARG),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=65, d=64, q=64, dff=64), sg.ERR_UNSUPPORTED),
    (dict(kind=sg.KIND_LAYERCHAIN, M=65, L=2, d=64, q=64, dff=64), sg.ERR_UNSUPPORTED),
    (dict(M=1, K=8, N=1), sg.OK),
    (dict(M=32, flags=sg.F_MTILE_ITEMS | sg.F_FORCE_DOT2), sg.ERR_INVALID_ARG),
    (dict(M=32, K=1024, N=1024, flags=sg.F_MTILE_ITEMS, ksl=2), sg.ERR_UNSUPPORTED),
    (dict(M=32, K=1024, N=1024, flags=sg.F_MTILE_ITEMS), sg.OK),
    (dict(kind=sg.KIND_LAYERCHAIN, M=32, L=2, d=64, q=64, dff=64, flags=sg.F_MTILE_ITEMS), sg.ERR_UNSUPPORTED),
    (dict(M=64, K=12288, N=4096), sg.OK),
    # a chain stage whose weight extent would pass 2 GiB (q_cols x d_model x 2 bytes)
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=1, d=32768, q=32768, dff=64), sg.ERR_UNSUPPORTED),
    (dict(kind=sg.KIND_LAYERCHAIN, M=4, L=1, d=64, q=64, dff=1 << 24), sg.ERR_UNSUPPORTED),
])
def test_plan_create_validation(kw, code):
    assert _create(**kw) == code


def test_forced_plans_of_the_gpu_parity_cases():
    """The forced split, K-slice and m-tile-item combinations the GPU parity
    tests run are accepted, and the ones they leave out are refused with
    SGEMM_ERR_UNSUPPORTED (X window or K-slice buffers past the LDS, or an
    empty slice), not silently replanned."""
    from helpers import KSL_CASES, KSL_REFUSED, MTI_CASES, MTI_REFUSED, SPLITK_SHAPES

    for M, K, N in SPLITK_SHAPES:
        for s in (2, 5, 11):
            assert sg.Gemm(M, K, N, splitk=s).describe()["stage"]["S"] > 1
    for M, K, N, ksl, s in KSL_CASES:
        assert sg.Gemm(M, K, N, kslices=ksl, splitk=s).describe()["stage"]["ksl"] == ksl
    for M, K, N, s in MTI_CASES:
        assert sg.Gemm(M, K, N, flags=sg.F_MTILE_ITEMS, splitk=s).describe()["stage"]["mtiles"] == -(-M // 16)
    for M, K, N, ksl, s in KSL_REFUSED:
        assert _create(M=M, K=K, N=N, ksl=ksl, splitk=s) == sg.ERR_UNSUPPORTED
    for M, K, N, s in MTI_REFUSED:
        assert _create(M=M, K=K, N=N, flags=sg.F_MTILE_ITEMS, splitk=s) == sg.ERR_UNSUPPORTED


# Static LDS a kernel may declare next to its planned dynamic region (the
# build refuses a kernel that declares more).
STATIC_LDS_RESERVE = 256


@pytest.mark.parametrize("d,q,dff", [(4096, 4096, 12288), (5120, 5120, 13824), (4096, 4096, 14336)])
@pytest.mark.parametrize("flags", [0, sg.F_SCHEDULER])
def test_chain_lds_fits_next_to_static_lds(d, q, dff, flags):
    """Every chain plan for M = 1..64 keeps its dynamic LDS within 160 KB minus
    the static-LDS reserve, so dynamic plus the kernel's own static LDS fits
    a CU."""
    for M in range(1, 65):
        for st in sg.LayerChain(M, 2, d, q, dff, flags=flags).describe()["stages"]:
            assert st["lds"] + STATIC_LDS_RESERVE <= 160 * 1024, (M, st)


@pytest.mark.parametrize("M", [1, 8, 16, 33, 44, 52, 64])
def test_gemm_lds_fits_next_to_static_lds(M):
    for K, N in ((4096, 6144), (4096, 24576), (12288, 4096), (7168, 1536), (5120, 13824)):
        st = sg.Gemm(M, K, N).describe()["stage"]
        assert st["lds"] + STATIC_LDS_RESERVE <= 160 * 1024, (M, K, N, st)


def test_build_refuses_kernels_with_more_static_lds():
    from chiplet_aware_persistent_amd import build

    assert build.STATIC_LDS_RESERVE == STATIC_LDS_RESERVE
    remarks = ("x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark:     LDS Size [bytes/block]: 16 [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark: Function Name: _Z1jv [-Rpass-analysis=kernel-resource-usage]\n"
               "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build.resource_usage(remarks, "LDS Size [bytes/block]") == {"_Z1kv": 16}
    assert build.scratch_usage(remarks) == {"_Z1jv": 8}


def test_device_check_without_a_device():
    """sgemm_device_check: a bad ordinal is an argument error; here no device
    can be queried (the call fails cleanly, nothing is cached); a run on a
    plan fails the same way before launching."""
    assert sg.sgemm_device_check(-1) == sg.ERR_INVALID_ARG
    assert sg.sgemm_device_check(64) == sg.ERR_INVALID_ARG
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except ImportError:
        has_gpu = False
    if not has_gpu:
        assert sg.sgemm_device_check(0) == sg.ERR_HIP
        g = sg.Gemm(4, 256, 128)
        assert sg.sgemm_run(g.handle, 16, 16, 16, 16) == sg.ERR_HIP


def test_binding_rejects_mismatched_tensors():
    torch = pytest.importorskip("torch")
    g = sg.Gemm(4, 256, 128)
    X = torch.zeros((4, 256), dtype=torch.bfloat16)
    W = torch.zeros((128, 256), dtype=torch.bfloat16)
    Y = torch.zeros((4, 128), dtype=torch.float32)
    ws = torch.zeros(g.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError):
        g(X, W, Y, ws[:-1])
    with pytest.raises(ValueError):
        g(X.float(), W, Y, ws)
    with pytest.raises(ValueError):
        g(X, W.t().contiguous().t(), Y, ws)
    with pytest.raises(ValueError):
        g(X, W, Y.to(torch.bfloat16), ws)
    ch = sg.LayerChain(2, 1, 64, 64, 64)
    Wq, Wo = torch.zeros((64, 64), dtype=torch.bfloat16), torch.zeros((64, 64), dtype=torch.bfloat16)
    Wgu, Wd = torch.zeros((128, 64), dtype=torch.bfloat16), torch.zeros((64, 64), dtype=torch.bfloat16)
    X0 = torch.zeros((2, 64), dtype=torch.bfloat16)
    Yf = torch.zeros((2, 64), dtype=torch.float32)
    cws = torch.zeros(ch.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ch(X0, [Wq], [Wo], [Wgu], [Wd], Yf, cws, Y_bf16=torch.zeros((2, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        ch(X0, [Wq], [Wo], [Wgu], [Wd], Yf, cws[:16])
    with pytest.raises(ValueError):
        ch(torch.zeros((2, 128), dtype=torch.bfloat16)[:, ::2], [Wq], [Wo], [Wgu], [Wd], Yf, cws)
    with pytest.raises(ValueError):
        ch(X0, [Wq, Wq], [Wo], [Wgu], [Wd], Yf, cws)


@pytest.mark.parametrize("M,K,N", [(16, 4096, 24576), (64, 4096, 24576), (64, 12288, 4096), (33, 2048, 1536),
                                   (64, 8, 1), (5, 1032, 777), (20, 12288, 300), (64, 4104, 129)])
@pytest.mark.parametrize("ntw,splitk", [(0, 0), (2, 3), (3, 0), (4, 0), (6, 2), (8, 0)])
def test_kchunk_plan_covers_columns_and_k(M, K, N, ntw, splitk):
    """K-chunked plans: blocks of 16 * tiles columns cover each XCD's columns,
    splits cover K in whole 512-wide chunks (a multiple of the ring depth per
    item), two X chunk buffers and the first round of the eight-wave
    reduction fit the LDS next to the static reserve."""
    MT = -(-M // 16)
    if ntw == 8 and MT > 2:
        assert _create(M=M, K=K, N=N, flags=sg.F_KCHUNK, tn=128, splitk=splitk) == sg.ERR_UNSUPPORTED
        return
    st = sg.Gemm(M, K, N, flags=sg.F_KCHUNK, tn=16 * ntw, splitk=splitk).describe()["stage"]
    assert st["path"] == "kc" and st["ta"] == MT and (ntw == 0 or st["tb"] == ntw)
    tiles = st["tb"]
    ring = 1 if tiles >= 6 else (2 if tiles >= 4 else 4)
    assert st["CB"] == 16 * tiles and st["NB"] * st["CB"] >= st["Nx"] and 8 * st["Nx"] >= N
    assert st["KS"] % (512 * ring) == 0 and st["steps"] * 512 == st["KS"]
    assert st["S"] * st["KS"] >= K and (st["S"] - 1) * st["KS"] < K
    assert st["items"] == st["NB"] * st["S"]
    rows = min(16 * MT, M + 1)
    assert st["xbuf"] >= rows * 520 * 2 and st["xbuf"] % 1024 == 0
    assert st["lds"] >= max(2 * st["xbuf"], 4 * tiles * MT * 1024)
    assert st["lds"] + STATIC_LDS_RESERVE <= 160 * 1024


@pytest.mark.parametrize("M,K,N", [(64, 4096, 24576), (48, 12288, 4096), (33, 2056, 900), (17, 776, 530),
                                   (64, 4096, 1536)])
@pytest.mark.parametrize("tm", [16, 32, 64])
@pytest.mark.parametrize("msplit", [False, True])
def test_mtile_window_and_msplit_plans(M, K, N, tm, msplit):
    """M-major window ablations: T_M-row windows per item (ceil(M / T_M) items
    per column block and split) in the m-tile-fastest order, and the M-split
    order (column block fastest).  The item count and the window rows cover
    every output row and column once."""
    flags = sg.F_MSPLIT if msplit else sg.F_MTILE_ITEMS
    st = sg.Gemm(M, K, N, flags=flags, tm=tm).describe()["stage"]
    assert st["path"] == "mfma" and st["ta"] == tm // 16
    assert st["mtiles"] == -(-M // tm) and st["nfast"] == (1 if msplit else 0)
    assert st["items"] == st["NB"] * st["S"] * st["mtiles"]
    assert st["mtiles"] * tm >= M and (st["mtiles"] - 1) * tm < M
    assert st["lds"] + STATIC_LDS_RESERVE <= 160 * 1024


def test_mtile_window_flag_combinations():
    assert _create(M=32, K=1024, N=1024, flags=sg.F_MTILE_ITEMS, tm=48) == sg.ERR_INVALID_ARG
    assert _create(M=32, K=1024, N=1024, tm=32) == sg.ERR_INVALID_ARG             # tm without the ablation
    assert _create(M=32, K=1024, N=1024, flags=sg.F_MSPLIT, tm=32) == sg.OK
    assert _create(kind=sg.KIND_LAYERCHAIN, M=32, L=2, d=64, q=64, dff=64, flags=sg.F_MSPLIT) == sg.ERR_UNSUPPORTED


def test_kchunk_flag_combinations():
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK | sg.F_FORCE_DOT2) == sg.ERR_INVALID_ARG
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK | sg.F_MTILE_ITEMS) == sg.ERR_INVALID_ARG
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK, ksl=2) == sg.ERR_UNSUPPORTED
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK, tn=40) == sg.ERR_UNSUPPORTED
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK, tn=80) == sg.ERR_UNSUPPORTED
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK, waves=4) == sg.ERR_UNSUPPORTED
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK, tn=64) == sg.OK


@pytest.mark.parametrize("M", [17, 24, 32, 33, 64])
@pytest.mark.parametrize("d,q,dff", [(4096, 4096, 12288), (256, 128, 384), (1032, 520, 1000)])
def test_chain_kchunk_plans(M, d, q, dff):
    """K-chunked chain stages (M = 17-32, two m-tiles): every stage on the
    path with one tile count for the unpaired stages, whole chunk groups per
    split; more m-tiles are refused (their kernels would not fit the
    registers next to the chain's state)."""
    MT = -(-M // 16)
    if MT != 2:
        assert _create(kind=sg.KIND_LAYERCHAIN, M=M, L=2, d=d, q=q, dff=dff, flags=sg.F_KCHUNK) == \
            sg.ERR_UNSUPPORTED
        return
    st = sg.LayerChain(M, 2, d, q, dff, flags=sg.F_KCHUNK).describe()["stages"]
    assert [s["path"] for s in st] == ["kc"] * 4 and all(s["ta"] == MT for s in st)
    assert st[0]["tb"] == st[1]["tb"] == st[3]["tb"] and st[2]["paired"] == 1 and st[2]["tb"] % 2 == 0
    for s, (K, N) in zip(st, ((d, q), (q, d), (d, dff), (dff, d))):
        tiles = s["tb"]
        ring = 1 if tiles >= 6 else (2 if tiles >= 4 else 4)
        assert s["ring"] == ring and s["KS"] % (512 * ring) == 0
        assert s["S"] * s["KS"] >= K and (s["S"] - 1) * s["KS"] < K
        np_ = tiles // 2 if s["paired"] else tiles
        assert s["CB"] == 16 * np_ and s["NB"] * s["CB"] >= s["Nx"] and 8 * s["Nx"] >= N
        assert s["lds"] + STATIC_LDS_RESERVE <= 160 * 1024


def test_chain_kchunk_flag_combinations():
    chain = dict(kind=sg.KIND_LAYERCHAIN, L=2, d=256, q=128, dff=384)
    assert _create(M=32, flags=sg.F_KCHUNK, **chain) == sg.OK
    assert _create(M=32, flags=sg.F_KCHUNK | sg.F_SCHEDULER, **chain) == sg.OK
    assert _create(M=16, flags=sg.F_KCHUNK, **chain) == sg.ERR_UNSUPPORTED     # one m-tile: not built
    assert _create(M=33, flags=sg.F_KCHUNK, **chain) == sg.ERR_UNSUPPORTED     # three: not built
    assert _create(M=32, flags=sg.F_KCHUNK | sg.F_FORCE_MFMA, **chain) == sg.ERR_UNSUPPORTED
    assert _create(M=32, flags=sg.F_KCHUNK, ksl=2, **chain) == sg.ERR_UNSUPPORTED
    assert _create(M=32, flags=sg.F_KCHUNK, waves=4, **chain) == sg.ERR_UNSUPPORTED
    assert _create(M=32, flags=sg.F_KCHUNK, tn=64, **chain) == sg.OK            # four tiles per item
    assert _create(M=32, flags=sg.F_KCHUNK, tn=96, **chain) == sg.ERR_UNSUPPORTED


@pytest.mark.parametrize("M,d,q,dff", [(1, 4096, 4096, 12288), (2, 4096, 4096, 12288), (2, 1024, 1032, 3000),
                                       (1, 256, 128, 384)])
def test_chain_lds_weight_prefetch_plans(M, d, q, dff, monkeypatch):
    """Ablation SGEMM_CHAIN_WPF: dot2 chain stages take whole ring groups of
    their first item's steps into LDS ahead of the wait, as many as fit next
    to the window and stash (eight waves x G kilobytes per step) up to the
    cap; off by default."""
    assert all(s["wpf"] == 0 for s in sg.LayerChain(M, 2, d, q, dff).describe()["stages"])  # off by default
    monkeypatch.setenv("SGEMM_CHAIN_WPF", "1000")
    st = sg.LayerChain(M, 2, d, q, dff).describe()["stages"]
    for s in st:
        assert s["path"] == "dot2" and s["wpf"] % s["ring"] == 0 and 0 < s["wpf"] <= s["steps"]
        assert s["lds"] + STATIC_LDS_RESERVE <= 160 * 1024
    if M == 1 and d == 4096:
        assert [s["wpf"] for s in st] == [8, 8, 8, 8]
    monkeypatch.setenv("SGEMM_CHAIN_WPF", "0")
    assert all(s["wpf"] == 0 for s in sg.LayerChain(M, 2, d, q, dff).describe()["stages"])
    monkeypatch.setenv("SGEMM_CHAIN_WPF", "-1")
    with pytest.raises(sg.SgemmError):
        sg.LayerChain(M, 2, d, q, dff)
    monkeypatch.delenv("SGEMM_CHAIN_WPF")
    monkeypatch.setenv("SGEMM_CHAIN_WPF", "1000")
    mf = sg.LayerChain(16, 2, d, q, dff).describe()["stages"]
    assert all(s["wpf"] == 0 for s in mf)  # MFMA stages: not used


@pytest.mark.parametrize("M,d,q,dff", [(1, 4096, 4096, 12288), (2, 1024, 1032, 3000), (2, 256, 128, 200),
                                       (8, 1024, 1024, 3072)])
def test_chain_and_decoder_round_robin_plans(M, d, q, dff, monkeypatch):
    """Chain and decoder dot2 stages with one K split take their items
    round-robin over the XCD's streams by default when a wave holds at most 16
    (column, row) sums; SGEMM_CHAIN_RR=0, an LDS weight prefetch or the
    scheduler mode keep contiguous ranges; a malformed value is refused."""
    monkeypatch.delenv("SGEMM_CHAIN_RR", raising=False)

    def want(s):
        fits = M * s["tb"] <= 16 if s["path"] == "dot2" else (s["path"] == "mfma" and s["mtiles"] == 1)
        return int(fits and s["S"] == 1 and s["wpf"] == 0)

    st = sg.LayerChain(M, 2, d, q, dff, flags=sg.F_FORCE_DOT2).describe()["stages"]
    assert [s["rr"] for s in st] == [want(s) for s in st]
    if M == 1 and d == 4096:
        assert all(s["rr"] == 1 for s in st)
    if M <= 2:  # the decoder's dot2 stages are built for M <= 2
        dec = sg.Decoder(M, 2, 1024, 3072, 8, 2, 128, 100).describe()["stages"]
        assert [s["rr"] for s in dec] == [want(s) for s in dec] and any(s["rr"] for s in dec)
    sch = sg.LayerChain(M, 2, d, q, dff, flags=sg.F_FORCE_DOT2 | sg.F_SCHEDULER).describe()["stages"]
    assert all(s["rr"] == 0 for s in sch)
    mf = sg.LayerChain(16, 2, d, q, dff).describe()["stages"]
    assert [s["rr"] for s in mf] == [int(s["path"] == "mfma" and s["mtiles"] == 1 and s["S"] == 1) for s in mf]
    monkeypatch.setenv("SGEMM_CHAIN_WPF", "1000")
    assert all(s["rr"] == 0 for s in sg.LayerChain(M, 2, d, q, dff, flags=sg.F_FORCE_DOT2).describe()["stages"])
    monkeypatch.delenv("SGEMM_CHAIN_WPF")
    monkeypatch.setenv("SGEMM_CHAIN_RR", "0")
    assert all(s["rr"] == 0 for s in sg.LayerChain(M, 2, d, q, dff, flags=sg.F_FORCE_DOT2).describe()["stages"])
    monkeypatch.setenv("SGEMM_CHAIN_RR", "1x")
    with pytest.raises(sg.SgemmError):
        sg.LayerChain(M, 2, d, q, dff)


def test_decoder_dot2_stages_take_four_columns(monkeypatch):
    """The decoder's dot2 stages (M <= 2) take four columns per wave unless
    the tile width is given (two is still allowed)."""
    monkeypatch.delenv("SGEMM_TN", raising=False)
    for M in (1, 2):
        st = sg.Decoder(M, 2, 4096, 12288, 32, 8, 128, 1024).describe()["stages"]
        assert [s["path"] for s in st] == ["dot2"] * 4 and all(s["tb"] == 4 for s in st)
    monkeypatch.setenv("SGEMM_TN", "2")
    st = sg.Decoder(1, 2, 4096, 12288, 32, 8, 128, 1024).describe()["stages"]
    assert all(s["tb"] == 2 for s in st)


def _stage_items(st, slots=32):
    """(slot, stream) -> item list of one chain/GEMM stage, as the kernels
    assign them: workgroup slot w of 32 runs streams q < ng, each the
    contiguous balanced range of the XCD's items (split-major)."""
    items, ng = st["items"], st["waves"] // st["wpi"]
    out = {}
    for w in range(slots):
        for q in range(ng):
            nw, ww = slots * ng, w * ng + q
            out[(w, q)] = list(range(items * ww // nw, items * (ww + 1) // nw))
    return out


@pytest.mark.parametrize("M,L,d,q,dff", [(2, 2, 256, 128, 200), (1, 36, 4096, 4096, 12288), (16, 3, 256, 128, 384),
                                         (64, 36, 4096, 4096, 12288), (8, 4, 512, 256, 1536), (5, 3, 256, 128, 384)])
def test_chain_stage_items_windows_and_shared_lines(M, L, d, q, dff):
    """Host model of how each chain stage's items fall to workgroups: every
    item runs exactly once; every K range a workgroup's items read lies in
    the one X window it stages for the stage (the window starts at its first
    item's split); and the per-XCD output columns of each stage tile the
    output.  It also lists how many XCDs write into each 128-byte line of
    each stage's output (the ragged 256-wide chain has two XCDs per line),
    the case the repeat test on the GPU exercises."""
    ch = sg.LayerChain(M, L, d, q, dff)
    outs = {0: q, 1: d, 2: dff, 3: d}
    for si, st in enumerate(ch.describe()["stages"]):
        assign = _stage_items(st)
        seen = sorted(i for v in assign.values() for i in v)
        assert seen == list(range(st["items"]))
        per_split = st["NB"] * st["mtiles"]
        kstep = 512 if st["path"] == "dot2" else 64
        for w in range(32):
            its = [i for qq in range(st["waves"] // st["wpi"]) for i in assign[(w, qq)]]
            if not its:
                continue
            s_first = min(its) // per_split
            for i in its:
                k0 = (i // per_split) * st["KS"]
                lo = k0 - s_first * st["KS"]
                hi = lo + (st["ksl"] - 1) * st["kss"] + st["steps"] * kstep
                assert 0 <= lo and hi <= st["win"], (si, w, i)
        # output columns: XCD x owns [x*Nx, (x+1)*Nx); count XCDs per 128-B line of a bf16 row
        N, Nx = outs[si], st["Nx"]
        owners = [min(c // Nx, 7) for c in range(N)]
        assert sorted(set(owners)) == list(range(min(8, -(-N // Nx))))
        per_line = [len(set(owners[c:c + 64])) for c in range(0, N, 64)]
        if (M, d) == (2, 256) and si == 3:
            assert max(per_line) == 2      # the down output x' of the ragged case: two XCDs per line


def _dec_create(M=4, L=2, d=256, dff=384, Hq=8, Hkv=2, hd=128, T=100, flags=0, q=0):
    p = sg.Problem(sg.KIND_DECODER, M, 0, 0, 0, L, d, q, dff, flags, 0, 0, 0, 0, 0, Hq, Hkv, hd, T)
    rc, h, ws = sg.sgemm_plan_create(p)
    if h:
        sg.sgemm_plan_destroy(h)
    return rc


def test_decoder_plan_validation():
    assert _dec_create() == sg.OK
    assert _dec_create(M=64, d=4096, dff=12288, Hq=32, Hkv=8, T=1024) == sg.OK
    assert _dec_create(Hq=6, Hkv=4) == sg.ERR_INVALID_ARG          # heads not a multiple
    assert _dec_create(Hq=16, Hkv=2) == sg.ERR_UNSUPPORTED         # 8 query heads per key/value head
    assert _dec_create(hd=64) == sg.ERR_UNSUPPORTED
    assert _dec_create(T=4096) == sg.ERR_UNSUPPORTED              # more than 64 chunks of 64
    assert _dec_create(T=4095) == sg.OK
    assert _dec_create(M=65) == sg.ERR_UNSUPPORTED
    assert _dec_create(d=100) == sg.ERR_INVALID_ARG
    assert _dec_create(q=999) == sg.ERR_INVALID_ARG
    assert _dec_create(q=1024) == sg.OK
    for f in (sg.F_SCHEDULER, sg.F_SYNC_FLAT, sg.F_POLL_LEADER, sg.F_LAUNCH_PER_STAGE, sg.F_KCHUNK, sg.F_MSPLIT):
        assert _dec_create(flags=f) == sg.ERR_UNSUPPORTED, f
    assert _dec_create(M=16, flags=sg.F_FORCE_DOT2) == sg.ERR_UNSUPPORTED


@pytest.mark.parametrize("M", [1, 2, 16, 64])
def test_decoder_plan_and_buffers(M):
    """Qwen3-8B-shaped decoder: QKV [4096 -> 6144], O [4096 -> 4096], paired
    gate_up [4096 -> 12288], down [12288 -> 4096]; per-layer activations that
    do not overlap; LDS within the CU: the widest stage (the attention stage
    takes 18 KB per wave: queries, weights and 64 value rows) plus the norm
    factors."""
    dec = sg.Decoder(M, 3, 4096, 12288, 32, 8, 128, 1024)
    dd = dec.describe()
    assert dd["kind"] == "decoder" and dd["chunks"] == 17
    # attention slices per (sequence, head) pair: fill an XCD's 32 workgroups (one head per XCD here)
    assert dd["attn_slices"] == {1: 8, 2: 8, 16: 2, 64: 1}[M]
    assert dd["lds"] >= 8 * (18 * 1024 + 512) + 256 and dd["lds"] + STATIC_LDS_RESERVE <= 160 * 1024
    st = dd["stages"]
    assert [(s["K"], s["N"]) for s in st] == [(4096, 6144), (4096, 4096), (4096, 12288), (12288, 4096)]
    assert st[2]["paired"] == 1
    assert {s["path"] for s in st} == {"dot2" if M <= 2 else "mfma"}
    assert all(s["lds"] + 256 + STATIC_LDS_RESERVE <= 160 * 1024 for s in st)
    spans = []
    cols = [6144, 4096, 4096, 12288, 4096]
    for l in range(3):
        for w in range(5):
            rc, off, nb = sg.sgemm_chain_buffer(dec.handle, l, w)
            assert rc == 0 and nb == M * cols[w] * 2 and off + nb <= dec.workspace_bytes and off % 16 == 0
            spans.append((off, off + nb))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert sg.sgemm_chain_buffer(dec.handle, 0, 5)[0] == sg.ERR_INVALID_ARG


def test_null_and_misaligned_arguments_rejected_before_launch():
    lib = sg.library()
    assert lib.sgemm_plan_create(None, 0, None, None) == sg.ERR_INVALID_ARG
    g = sg.Gemm(4, 256, 128)
    h = g.handle
    assert sg.sgemm_run(h, 0, 16, 16, 16) == sg.ERR_INVALID_ARG
    assert sg.sgemm_run(h, 16, 0, 16, 16) == sg.ERR_INVALID_ARG
    assert sg.sgemm_run(h, 16, 16, 16, 0) == sg.ERR_INVALID_ARG
    assert sg.sgemm_run(h, 18, 16, 16, 16) == sg.ERR_INVALID_ARG   # misaligned X
    assert sg.sgemm_run(h, 16, 24, 16, 16) == sg.ERR_INVALID_ARG   # misaligned W
    assert sg.sgemm_run(None, 16, 16, 16, 16) == sg.ERR_INVALID_ARG
    assert sg.layerchain_run(h, 16, [16], [16], [16], [16], 16, 0, 16) == sg.ERR_INVALID_ARG  # kind
    assert sg.sgemm_workspace_init(h, 0) == sg.ERR_INVALID_ARG
    assert lib.sgemm_topology_probe(None, 4, None) == sg.ERR_INVALID_ARG
    assert sg.status_string(sg.ERR_TIMEOUT) == "device wait timed out"


SHAPES = [(1, 1024, 1024), (1, 4096, 6144), (1, 4096, 4096), (1, 4096, 24576), (1, 12288, 4096),
          (8, 4096, 6144), (16, 4096, 4096), (32, 4096, 24576), (64, 12288, 4096), (1, 7168, 1536),
          (2, 7168, 4096), (16, 7168, 18432), (3, 520, 1000), (17, 776, 530), (5, 8, 17), (64, 8, 1),
          (64, 4096, 24576), (48, 4096, 24576)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_dot2_round_robin_items_cover_each_item_once(M, K, N, monkeypatch):
    """Single-launch dot2 and MFMA plans with one K split take their items
    round-robin over the XCD's 32 x ng streams (rr = 1; SGEMM_DOT2_RR=0 and
    SGEMM_MFMA_RR=0 give contiguous ranges, the K-chunked path, m-tile items
    and split plans always do): a host model of both
    assignments runs every item exactly once, and the longest stream is no
    longer than with contiguous ranges."""
    for env in ("1", "0"):
        monkeypatch.setenv("SGEMM_DOT2_RR", env)
        monkeypatch.setenv("SGEMM_MFMA_RR", env)
        st = sg.Gemm(M, K, N).describe()["stage"]
        rr_path = st["path"] == "dot2" or (st["path"] == "mfma" and st["mtiles"] == 1)
        if st["path"] == "lt":  # the large-tile path always takes its items round-robin
            assert st["rr"] == 1
        else:
            assert st["rr"] == (1 if env == "1" and rr_path and st["S"] == 1 else 0)
        items, ng = st["items"], st["waves"] // st["wpi"]
        nw = 32 * ng
        contiguous = [list(range(items * w // nw, items * (w + 1) // nw)) for w in range(nw)]
        streams = [list(range(w, items, nw)) for w in range(nw)] if st["rr"] else contiguous
        assert sorted(i for s_ in streams for i in s_) == list(range(items))
        assert max(len(s_) for s_ in streams) <= max(len(s_) for s_ in contiguous)
    with pytest.raises(sg.SgemmError):
        monkeypatch.setenv("SGEMM_DOT2_RR", "x")
        sg.Gemm(1, 1024, 1024)


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("splitk", [0, 3])
@pytest.mark.parametrize("flags", [0, sg.F_MTILE_ITEMS])
def test_planner_covers_every_column_and_k_once(M, K, N, splitk, flags):
    if flags and M < 16:
        return
    try:
        g = sg.Gemm(M, K, N, splitk=splitk, flags=flags)
    except sg.SgemmError as e:
        # a forced split count whose X window exceeds the LDS budget is refused
        assert splitk and e.code == sg.ERR_UNSUPPORTED
        return
    st = g.describe()["stage"]
    if st["path"] == "kc":   # long K or M > 48, wide N: the K-chunked path (its own coverage test below)
        assert M >= 16 and (K >= 6144 or M > 48) and not flags and not splitk and st["S"] == 1
        return
    if st["path"] == "lt":   # M > 48 with N or K >= 12288: 64 x 96 large tiles (their own coverage test)
        assert M > 48 and (N >= 12288 or K >= 12288) and not flags and not splitk
        _check_large_tile_plan(st, M, K, N, 4)
        assert 32 * st["ta"] == 64 and st["CB"] == 96
        return
    assert st["path"] == ("dot2" if M < 16 else "mfma")
    mt = st["mtiles"]
    assert mt == (math.ceil(M / 16) if flags else 1) and (mt == 1 or st["ta"] == 1)
    assert 16 * st["ta"] * mt >= M                     # m-tiles cover every row
    Nx, CB, NB, S, KS = st["Nx"], st["CB"], st["NB"], st["S"], st["KS"]
    ksl, kss = st["ksl"], st["kss"]
    assert st["wpi"] % ksl == 0 and CB == st["wpi"] // ksl * st["TN"] and st["waves"] % st["wpi"] == 0
    assert ksl == 1 or (st["path"] == "mfma" and st["wpi"] == st["waves"])  # one item stream per workgroup
    assert 8 * Nx >= N and 8 * (Nx - 16) < N          # per-XCD partition covers N, no spare XCD block
    assert NB * CB >= Nx                               # column blocks cover the XCD's columns
    assert S * KS >= K and (S - 1) * KS < K            # splits cover K, none empty
    assert ksl * kss >= KS and (ksl - 1) * kss < KS    # slices cover a split, none empty
    assert KS % 64 == 0 and st["items"] == NB * S * mt  # splits start on 128-byte lines
    kstep = 512 if st["path"] == "dot2" else 64
    assert ksl == 1 or kss % kstep == 0
    assert st["steps"] * kstep >= kss
    assert st["lds"] <= 160 * 1024
    # every k of a split is streamed by exactly one slice, and the LDS window
    # holds what the last slice reads including its padded steps
    for s in range(S):
        seen = []
        for q in range(ksl):
            k0 = s * KS + q * kss
            klim = min(min(K, (s + 1) * KS) - k0, kss)
            seen += list(range(k0, k0 + max(klim, 0)))
        assert seen == list(range(s * KS, min(K, (s + 1) * KS)))
    assert st["win"] >= (ksl - 1) * kss + st["steps"] * kstep
    if splitk:
        assert S == math.ceil(K / (math.ceil(math.ceil(K / splitk) / 64) * 64))
    # columns: every column owned by exactly one (xcd, block, wave, lane-column)
    owned = set()
    for x in range(8):
        for b in range(NB):
            for c in range(CB):
                col = x * Nx + b * CB + c
                if x * Nx + b * CB + c < min(N, (x + 1) * Nx) and b * CB + c < Nx:
                    assert col not in owned
                    owned.add(col)
    assert owned == set(range(N))


def test_chain_plan_and_buffers():
    c = sg.LayerChain(64, 36, 4096, 4096, 12288)
    d = c.describe()
    assert d["kind"] == "layerchain" and len(d["stages"]) == 4
    assert d["stages"][2]["paired"] == 1 and d["stages"][2]["N"] == 12288
    spans = []
    for l in (0, 17, 35):
        for w in range(4):
            rc, off, nb = sg.sgemm_chain_buffer(c.handle, l, w)
            assert rc == 0 and off + nb <= c.workspace_bytes and off % 16 == 0
            spans.append((off, off + nb))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert sg.sgemm_chain_buffer(c.handle, 36, 0)[0] == sg.ERR_INVALID_ARG
    assert sg.sgemm_chain_buffer(c.handle, 0, 4)[0] == sg.ERR_INVALID_ARG


def test_chain_path_choice():
    """dot2 stages at M <= 2 (G weight rows per wave, gate_up holding G/2
    gate/up pairs), MFMA stages above; SGEMM_F_FORCE_DOT2 (M < 16) and
    SGEMM_F_FORCE_MFMA choose the path, and FORCE_DOT2 is refused at M >= 16."""
    def paths(M, flags=0):
        return [s["path"] for s in sg.LayerChain(M, 4, 4096, 4096, 12288, flags=flags).describe()["stages"]]
    for M, flags in ((1, 0), (2, 0), (3, sg.F_FORCE_DOT2), (8, sg.F_FORCE_DOT2), (15, sg.F_FORCE_DOT2)):
        st = sg.LayerChain(M, 4, 4096, 4096, 12288, flags=flags).describe()["stages"]
        assert [s["path"] for s in st] == ["dot2"] * 4, M
        g = st[0]["tb"]
        assert g in (2, 4) and all(s["tb"] == g for s in st) and g * M <= 64
        assert st[2]["paired"] == 1 and st[2]["TN"] == g // 2 and st[0]["TN"] == g
    for M in (3, 8, 15, 16, 17, 64):
        assert paths(M) == ["mfma"] * 4, M
    assert paths(1, sg.F_FORCE_MFMA) == ["mfma"] * 4
    with pytest.raises(sg.SgemmError):
        sg.LayerChain(16, 4, 4096, 4096, 12288, flags=sg.F_FORCE_DOT2)


def test_chain_scheduler_plan():
    """With SGEMM_F_SCHEDULER the stages are planned over 31 worker slots per
    XCD (slot 0 schedules); the grid stays 8 x 32.  The mode is a chain runtime:
    refused for a single GEMM and with the flat or poll-leader counters."""
    for M in (1, 16, 64):
        base = sg.LayerChain(M, 4, 4096, 4096, 12288).describe()
        sch = sg.LayerChain(M, 4, 4096, 4096, 12288, flags=sg.F_SCHEDULER).describe()
        assert sch["grid"] == base["grid"] == 256
        assert [s["slots"] for s in base["stages"]] == [32] * 4
        assert [s["slots"] for s in sch["stages"]] == [31] * 4
        assert [s["path"] for s in sch["stages"]] == [s["path"] for s in base["stages"]]
    for flags in (sg.F_SCHEDULER | sg.F_SYNC_FLAT, sg.F_SCHEDULER | sg.F_POLL_LEADER):
        with pytest.raises(sg.SgemmError):
            sg.LayerChain(16, 4, 4096, 4096, 12288, flags=flags)
    with pytest.raises(sg.SgemmError):
        sg.Gemm(16, 4096, 4096, flags=sg.F_SCHEDULER)


def test_eq1_matches_the_pages_table():
    g = json.load(open(os.path.join(GOLD, "eq1_l2_hit.json")))
    for row in g["rows"]:
        assert model.eq1_hit(row["B"], W=g["W"], T_M=g["T_M"]) == pytest.approx(row["predicted_hit"])
    assert model.eq1_hit(10 ** 6, W=g["W"]) == pytest.approx(g["limit_hit_W31"], abs=1e-4)
    ex = g["ai_eff_example"]
    assert model.ai_eff(ex["B"], ex["hit"]) == pytest.approx(ex["ai_eff_approx"], rel=0.02)


def test_roofline_floors():
    # 2*K*N bytes at 8 TB/s: QKV 4096x6144 -> 6.29 us, down 12288x4096 -> 12.58 us
    assert model.floor_us(4096, 6144) == pytest.approx(6.29, abs=0.01)
    assert model.floor_us(12288, 4096) == pytest.approx(12.58, abs=0.01)
    assert model.ridge_flop_per_byte() == pytest.approx(312.5)


def test_build_reads_scratch_usage_from_compiler_remarks():
    from chiplet_aware_persistent_amd import build
    remarks = "\n".join([
        "x.hip:14:1: remark: Function Name: _ZN2sg4k_aEv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:14:1: remark:     VGPRs: 105 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:14:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:21:1: remark: Function Name: _ZN2sg4k_bEv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:21:1: remark:     ScratchSize [bytes/lane]: 3136 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.scratch_usage(remarks) == {"_ZN2sg4k_aEv": 0, "_ZN2sg4k_bEv": 3136}


def test_read_probe_rejects_bad_arguments_before_launch():
    lib = sg.library()
    assert lib.sgemm_read_probe(None, 1024, 0, 16, 256, None) == sg.ERR_INVALID_ARG
    assert lib.sgemm_read_probe(16, 1024, 0, None, 256, None) == sg.ERR_INVALID_ARG
    assert lib.sgemm_read_probe(24, 1024, 0, 16, 256, None) == sg.ERR_INVALID_ARG    # misaligned source
    assert lib.sgemm_read_probe(16, 1024, 0, 18, 256, None) == sg.ERR_INVALID_ARG    # misaligned sink
    assert lib.sgemm_read_probe(16, 1000, 0, 16, 256, None) == sg.ERR_INVALID_ARG    # not whole 16-byte chunks
    assert lib.sgemm_read_probe(16, 1 << 31, 0, 16, 256, None) == sg.ERR_INVALID_ARG  # past the buffer extent
    assert lib.sgemm_read_probe(16, 1024, 2, 16, 256, None) == sg.ERR_INVALID_ARG    # pattern
    assert lib.sgemm_read_probe(16, 1024, 0, 16, 12, None) == sg.ERR_INVALID_ARG     # grid not a multiple of 8
    assert lib.sgemm_read_probe(16, 1024, 0, 16, 8192, None) == sg.ERR_INVALID_ARG


@pytest.mark.parametrize("name,value,kind", [
    ("SGEMM_SPLITK", "two", sg.KIND_GEMM), ("SGEMM_WAVES", "6", sg.KIND_GEMM), ("SGEMM_KSLICES", "3", sg.KIND_GEMM),
    ("SGEMM_TN", "-1", sg.KIND_GEMM), ("SGEMM_WATCHDOG_S", "abc", sg.KIND_LAYERCHAIN),
    ("SGEMM_WATCHDOG_S", "0", sg.KIND_LAYERCHAIN), ("SGEMM_CHAIN_COST", "1.5,75", sg.KIND_LAYERCHAIN),
    ("SGEMM_CHAIN_COST", "0.5,75,0.5,0.05,0.25", sg.KIND_LAYERCHAIN), ("SGEMM_CHAIN_S", "1,2", sg.KIND_LAYERCHAIN)])
def test_malformed_environment_overrides_are_rejected(monkeypatch, name, value, kind):
    monkeypatch.setenv(name, value)
    if kind == sg.KIND_GEMM:
        assert _create(M=16, K=1024, N=1024) == sg.ERR_INVALID_ARG
    else:
        assert _create(kind=kind, M=4, L=2, d=256, q=128, dff=384) == sg.ERR_INVALID_ARG


def test_environment_overrides_apply(monkeypatch):
    monkeypatch.setenv("SGEMM_SPLITK", "4")
    monkeypatch.setenv("SGEMM_WATCHDOG_S", "2.5")
    assert sg.Gemm(16, 4096, 1024).describe()["stage"]["S"] == 4
    assert _create(kind=sg.KIND_LAYERCHAIN, M=4, L=2, d=256, q=128, dff=384) == sg.OK


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_is_plain_c_and_cpp(tmp_path, lang, compiler):
    """include/sgemm.h compiles on its own as C and as C++ (no HIP types)."""
    import shutil
    import subprocess

    if not shutil.which(compiler):
        pytest.skip(compiler + " not found")
    src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "sgemm.h"\nint main(void) { return SGEMM_F_MTILE_ITEMS != 0 ? 0 : 1; }\n')
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run([compiler, "-std=c11" if lang == "c" else "-std=c++17", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", inc, str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_python_constants_match_the_header(tmp_path):
    """Every SGEMM_* enumerator of include/sgemm.h has the same value in the
    binding (flags, status codes, kinds, output types)."""
    import re
    import shutil
    import subprocess

    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    header = open(os.path.join(inc, "sgemm.h")).read()
    names = sorted(set(re.findall(r"\b(SGEMM_(?:F|ERR|KIND|OUT)_[A-Z0-9_]+|SGEMM_OK)\s*=", header)))
    assert len(names) > 15
    src = tmp_path / "c.c"
    src.write_text('#include <stdio.h>\n#include "sgemm.h"\nint main(void) {\n' +
                   "".join('  printf("%s %%lld\\n", (long long)%s);\n' % (n, n) for n in names) + "  return 0;\n}\n")
    exe = tmp_path / "c"
    r = subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        name, value = line.split()
        py = name[len("SGEMM_"):]
        assert hasattr(sg, py), name
        assert getattr(sg, py) == int(value), (name, getattr(sg, py), value)


def test_chain_stamps_breakdown_on_a_made_up_timeline():
    """Two workgroups and five events (Q, O, gate_up and down of one layer,
    then Q of the next); every figure is worked out by hand below."""
    import numpy as np
    from chiplet_aware_persistent_amd.chain_stamps import stage_breakdown
    st = np.zeros((2, 5, 2))
    t = 0.0
    for e in range(5):
        st[0, e] = (t + 1.0, t + 5.0)   # workgroup 0 starts 1 us after the barrier, works 4 us
        st[1, e] = (t + 2.0, t + 8.0)   # workgroup 1 starts 2 us after, works 6 us
        t += 8.0
    b = stage_breakdown(st)
    assert set(b) == {"Q", "O", "gate_up", "down"}
    # release: first start (t+1) minus the previous last end (t)
    # skew 1; med_start 0.5; work_med 5; tail: 8 - median(5, 8) = 1.5; span: 8 - 1 = 7
    for v in b.values():
        assert v == [1.0, 1.0, 0.5, 5.0, 1.5, 7.0]


def test_bench_cpu_baselines_report_the_contract_fields():
    """Both workloads' CPU baselines time the oracle as it stands and say what
    they timed (tiny shapes here; the bench uses the full ones)."""
    import bench
    import synth
    x = synth.normal_bf16(1, 2, 256)
    ws = [synth.uniform_bf16(2, 128, 256, 0.05), synth.uniform_bf16(3, 256, 128, 0.05),
          synth.uniform_bf16(4, 2 * 384, 256, 0.05), synth.uniform_bf16(5, 256, 384, 0.05)]
    r = bench.cpu_baseline_chain(2, x, ws)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0 and r["cores"] >= 1
    assert "M=2" in r["sample"]


@pytest.mark.parametrize("M", [65, 80, 100, 127, 128, 129, 192, 200, 255, 256])
@pytest.mark.parametrize("K,N", [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096), (7168, 18432),
                                 (1032, 777), (8, 1)])
def test_large_m_plans_cover_rows_columns_and_k(M, K, N):
    """M = 65..256: the K-chunked path in 64-row m-blocks, items (split,
    block, m-block) taken round-robin.  A host walk of every (XCD, slot)
    pair's items covers every (m-block, column block, split) exactly once;
    the m-blocks cover the M rows, the blocks each XCD's columns and the
    splits K; LDS fits next to the static reserve."""
    st = sg.Gemm(M, K, N, flags=sg.F_KCHUNK).describe()["stage"]
    MB = -(-M // 64)
    assert st["path"] == "kc" and st["ta"] == 4 and st["mb"] == MB and st["rr"] == 1
    assert st["items"] == st["NB"] * st["S"] * MB
    assert st["NB"] * st["CB"] >= st["Nx"] and 8 * st["Nx"] >= N
    assert st["S"] * st["KS"] >= K and (st["S"] - 1) * st["KS"] < K
    assert (MB - 1) * 64 < M <= MB * 64
    assert st["xbuf"] >= 64 * 520 * 2 and st["lds"] + STATIC_LDS_RESERVE <= 160 * 1024
    seen = np.zeros(st["items"], dtype=np.int64)
    for slot in range(32):
        for it in range(slot, st["items"], 32):
            seen[it] += 1
    assert np.all(seen == 1)
    per_split = st["NB"] * MB
    triples = {(it // per_split, (it % per_split) // MB, it % MB) for it in range(st["items"])}
    assert len(triples) == st["items"]
    # round-robin: the m-blocks of one (split, block) are consecutive items, so
    # they land on consecutive slots of the XCD and run together
    for it in range(0, st["items"], MB):
        assert {(it + q) % MB for q in range(MB)} == set(range(MB))


def test_large_m_refusals():
    assert _create(M=257) == sg.ERR_UNSUPPORTED
    for fl in (sg.F_FORCE_MFMA, sg.F_MTILE_ITEMS, sg.F_MSPLIT, sg.F_W_SC1, sg.F_FORCE_DOT2):
        assert _create(M=65, K=1024, N=1024, flags=fl) == sg.ERR_UNSUPPORTED, fl
    # large tiles: nt weight loads with one m-block, the default policy when
    # several m-blocks share the weights (or when asked for)
    assert sg.Gemm(128, 4096, 24576, tm=128).describe()["w_aux"] == 2      # one 128-row m-block
    assert sg.Gemm(128, 4096, 24576).describe()["w_aux"] == 0              # two 64-row m-blocks
    assert sg.Gemm(256, 4096, 24576).describe()["w_aux"] == 0
    assert sg.Gemm(128, 4096, 24576, tm=128, flags=sg.F_W_CACHED).describe()["w_aux"] == 0
    assert _create(M=65, K=1024, N=1024, flags=sg.F_KCHUNK | sg.F_W_CACHED) == sg.ERR_UNSUPPORTED
    # the K-chunked kernels are built with nontemporal weight loads only
    assert _create(M=32, K=1024, N=1024, flags=sg.F_KCHUNK | sg.F_W_CACHED) == sg.ERR_UNSUPPORTED
    assert _create(M=64, K=4096, N=24576, flags=sg.F_W_CACHED) == sg.OK
    assert sg.Gemm(64, 4096, 24576, flags=sg.F_W_CACHED).describe()["stage"]["path"] == "mfma"
    assert sg.Gemm(64, 4096, 24576).describe()["stage"]["path"] == "lt"
    assert sg.Gemm(64, 12288, 4096).describe()["stage"]["path"] == "lt"
    assert sg.Gemm(64, 4096, 4096).describe()["stage"]["path"] == "mfma"
    assert sg.Gemm(48, 4096, 24576).describe()["stage"]["path"] == "mfma"
    assert _create(kind=sg.KIND_LAYERCHAIN, M=65, L=2, d=64, q=64, dff=64) == sg.ERR_UNSUPPORTED
    # large-tile path: tile widths are multiples of 32 columns, four waves, no K slices
    assert _create(M=65, K=1024, N=1024, tn=48) == sg.ERR_UNSUPPORTED
    assert _create(M=65, K=1024, N=1024, waves=2) == sg.ERR_INVALID_ARG      # 4 or 8 waves only
    assert _create(M=65, K=1024, N=1024, waves=8, tn=96) == sg.ERR_UNSUPPORTED   # 8 waves: 192 or 384
    assert _create(M=65, K=1024, N=1024, waves=8, tn=192) == sg.OK
    assert _create(M=65, K=1024, N=1024, ksl=2) == sg.ERR_UNSUPPORTED
    assert _create(M=65, K=1024, N=1024, tn=96) == sg.OK


@pytest.mark.parametrize("M", [65, 80, 100, 127, 128, 129, 192, 200, 255, 256])
@pytest.mark.parametrize("K,N", [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096), (7168, 18432),
                                 (1032, 777), (8, 1)])
def test_large_tile_plans_cover_rows_columns_and_k(M, K, N):
    """M = 65..256, default plans and plans forced to four or eight waves: the
    large-tile path (tiles of 32 MW rows x 16 NW x waves/2 columns), items
    (split, block, m-block) round-robin;
    the m-blocks cover M, the blocks each XCD's columns, the splits K in
    whole 32-wide steps, padded to the register ring depth; the two LDS
    buffers fit next to the static reserve; the loads in flight fit vmcnt."""
    for waves in (0, 4, 8):
        _check_large_tile_plan(sg.Gemm(M, K, N, waves=waves).describe()["stage"], M, K, N, waves)


def _check_large_tile_plan(st, M, K, N, waves):
    MW, NW, WV = st["ta"], st["tb"], st["waves"]
    assert st["path"] == "lt" and WV in (4, 8) and (waves == 0 or WV == waves) and st["rr"] == 1
    TM = 32 * MW
    assert st["mb"] == -(-M // TM) and (st["mb"] - 1) * TM < M
    assert st["CB"] == 16 * NW * (WV // 2) and st["NB"] * st["CB"] >= st["Nx"] and 8 * st["Nx"] >= N
    F = 2 * MW + (WV // 2) * NW  # two-kilobyte blocks per 64-wide K step
    LPW = -(-2 * F // WV)        # 16-byte loads per lane and step (two per block)
    D = max(2, min(8, (24 // LPW) // 2 * 2))  # steps in flight in registers (even)
    assert st["ring"] == D and LPW * (D - 1) < 64
    assert st["KS"] % 64 == 0 and st["steps"] % D == 0 and 0 <= st["steps"] * 64 - st["KS"] < 64 * D
    assert st["S"] * st["KS"] >= K and (st["S"] - 1) * st["KS"] < K
    assert st["items"] == st["NB"] * st["S"] * st["mb"]
    assert st["lds"] == 2 * F * 2048 and st["lds"] + STATIC_LDS_RESERVE <= 160 * 1024


@pytest.mark.parametrize("M", [1, 16, 33, 64])
def test_plans_up_to_64_rows_keep_one_m_block(M):
    """Below 65 rows nothing changes: one m-block and, on the K-chunked path,
    contiguous item ranges."""
    st = sg.Gemm(M, 4096, 24576, flags=sg.F_KCHUNK).describe()["stage"]
    assert st["mb"] == 1 and st["rr"] == 0 and st["items"] == st["NB"] * st["S"]


def _stage(M, K, N, **kw):
    return sg.Gemm(M, K, N, **kw).describe()["stage"]


def test_large_tile_environment_switches(monkeypatch):
    """SGEMM_LT=0 sends M = 65..256 to the K-chunked path; SGEMM_LT_MIN_M
    moves the fewest rows that take the large-tile path (never below 16);
    SGEMM_KC_RR=0 gives m-block plans contiguous item ranges; a malformed
    value of any of them is refused with SGEMM_ERR_INVALID_ARG."""
    for var in ("SGEMM_LT", "SGEMM_LT_MIN_M", "SGEMM_KC_RR"):
        monkeypatch.delenv(var, raising=False)
    assert _stage(128, 4096, 24576)["path"] == "lt"
    assert _stage(32, 4096, 4096)["path"] == "mfma"
    monkeypatch.setenv("SGEMM_LT", "0")
    st = _stage(128, 4096, 24576)
    assert st["path"] == "kc" and st["mb"] == 2
    monkeypatch.delenv("SGEMM_LT")
    monkeypatch.setenv("SGEMM_LT_MIN_M", "16")
    assert _stage(16, 4096, 4096)["path"] == "lt"
    assert _stage(15, 4096, 4096)["path"] == "dot2"
    monkeypatch.setenv("SGEMM_LT_MIN_M", "4")   # clamped to 16 rows
    assert _stage(8, 4096, 4096)["path"] == "dot2"
    monkeypatch.setenv("SGEMM_LT_MIN_M", "200")
    assert _stage(128, 4096, 24576)["path"] == "kc"
    assert _stage(200, 4096, 24576)["path"] == "lt"
    monkeypatch.delenv("SGEMM_LT_MIN_M")
    for kw in ({}, {"flags": sg.F_KCHUNK}):
        assert _stage(256, 4096, 24576, **kw)["rr"] == 1
    monkeypatch.setenv("SGEMM_KC_RR", "0")
    for kw in ({}, {"flags": sg.F_KCHUNK}):
        assert _stage(256, 4096, 24576, **kw)["rr"] == 0
    monkeypatch.delenv("SGEMM_KC_RR")
    for var in ("SGEMM_LT", "SGEMM_LT_MIN_M", "SGEMM_KC_RR"):
        monkeypatch.setenv(var, "1x")
        with pytest.raises(sg.SgemmError) as e:
            sg.Gemm(256, 4096, 24576)
        assert e.value.code == sg.ERR_INVALID_ARG, var
        monkeypatch.delenv(var)


def test_counter_copies_and_attention_slices_switches(monkeypatch):
    """SGEMM_CHAIN_GCOPIES takes 8 (one counter copy per XCD) or 1;
    SGEMM_ATTN_SLICES sets the decoder's attention slices (1..8); other
    values are refused with SGEMM_ERR_INVALID_ARG."""
    monkeypatch.delenv("SGEMM_CHAIN_GCOPIES", raising=False)
    monkeypatch.delenv("SGEMM_ATTN_SLICES", raising=False)
    for v, rc in (("8", sg.OK), ("1", sg.OK), ("2", sg.ERR_INVALID_ARG), ("x", sg.ERR_INVALID_ARG)):
        monkeypatch.setenv("SGEMM_CHAIN_GCOPIES", v)
        assert _dec_create() == rc, v
        p = sg.Problem(sg.KIND_LAYERCHAIN, 2, 0, 0, 0, 2, 256, 128, 384, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0)
        prc, h, ws = sg.sgemm_plan_create(p)
        if h:
            sg.sgemm_plan_destroy(h)
        assert prc == rc, v
    monkeypatch.delenv("SGEMM_CHAIN_GCOPIES")
    assert sg.Decoder(4, 2, 256, 384, 8, 2, 128, 100).describe()["attn_slices"] > 1
    for v in ("1", "3", "8"):
        monkeypatch.setenv("SGEMM_ATTN_SLICES", v)
        assert sg.Decoder(4, 2, 256, 384, 8, 2, 128, 100).describe()["attn_slices"] == int(v)
    for v in ("0", "9", "x"):
        monkeypatch.setenv("SGEMM_ATTN_SLICES", v)
        assert _dec_create() == sg.ERR_INVALID_ARG, v


@pytest.mark.parametrize("M", [1, 16, 64, 128, 256])
def test_decode_shapes_fit_the_no_alloc_array(M):
    """Every decode projection shape up to M = 256 plans a workspace (split-K
    counters, partials and control words together) below the 31 MiB that
    sgemm_run_noalloc's static array leaves for partials."""
    for K, N in [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096),
                 (7168, 1536), (7168, 4096), (7168, 18432)]:
        assert sg.Gemm(M, K, N).describe()["workspace"] < 31 * 2**20, (M, K, N)


def test_measured_split_rules():
    """MFMA, M = 17-48 on K = 4096 with at most 4096 columns: four K splits (a
    64 KB X window per workgroup).  dot2, M = 10-15, K = 6144-8192, 3072-4096
    columns: two splits where the cost model takes more.  Neighbouring shapes
    and forced splits keep the cost model's or the caller's choice."""
    for M in (17, 24, 32, 33, 36, 48):
        for N in (2048, 4096):
            st = _stage(M, 4096, N)
            assert st["path"] == "mfma" and st["S"] == 4 and st["KS"] == 1024, (M, N)
    assert _stage(16, 4096, 4096)["S"] == 1
    assert _stage(20, 3072, 4096)["S"] == 1
    assert _stage(32, 4096, 6144)["S"] == 2
    assert _stage(32, 4096, 4096, splitk=2)["S"] == 2
    for M, K, N in ((10, 7168, 3072), (12, 7168, 4096), (15, 7168, 4096), (15, 8192, 4096), (15, 6144, 4096)):
        st = _stage(M, K, N)
        assert st["path"] == "dot2" and st["S"] == 2, (M, K, N)
    assert _stage(12, 6144, 4096)["S"] == 1
    assert _stage(15, 7168, 1536)["S"] == 4
    assert _stage(8, 12288, 4096)["S"] == 4
    assert _stage(12, 7168, 4096, splitk=4)["S"] == 4
