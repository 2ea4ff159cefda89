"""GPU parity of the single decode GEMM (sgemm_run) against the CPU oracle.

Small shapes (spanning several tiles and ragged tails) and the configuration
shapes at full size (in the launch configuration the bench uses) are checked
element by element, every output element.  Exactness pins (integers,
all-ones, one-hot, powers of two, run-to-run determinism) are bitwise.
Every call goes through the C ABI (ctypes) into libsgemm.so.
"""
import numpy as np
import pytest

import chiplet_aware_persistent_amd as sg
import oracle
import synth
from helpers import (KSL_CASES, MTI_CASES, SPLITK_SHAPES, check, device_tensor_bf16, device_weights_checked,
                     gemm_inputs, host_bits, report)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run(g: sg.Gemm, X, W, ws=None):
    dev = X.device
    Y = torch.empty((g.M, g.N), dtype=torch.float32 if g.out_dtype == sg.OUT_F32 else torch.bfloat16,
                    device=dev)
    if ws is None:
        ws = g.new_workspace()
    g(X, W, Y, ws)
    rc = g.status(ws)
    assert rc == sg.OK, sg.status_string(rc)
    return Y


def _rotation(ids):
    """r when workgroup i ran on XCD (i + r) mod 8 for every i, else None."""
    r = {(x - i) % 8 for i, x in enumerate(ids)}
    return r.pop() if len(r) == 1 and all(0 <= x < 8 for x in ids) else None


def test_topology_is_round_robin(cuda_device):
    """Workgroups go to the 8 XCDs round-robin from some starting XCD, in eager
    launches on two streams and in graph replays (which move the starting
    XCD): the kernels index work by (hardware XCD, i / 8), which needs exactly
    this."""
    ids = sg.topology(256)
    assert sorted(set(ids)) == list(range(8))
    assert _rotation(ids) is not None, ids[:32]
    out = torch.full((256,), -1, dtype=torch.int32, device=cuda_device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert sg.sgemm_topology_probe(out.data_ptr(), 256, sg._stream_handle(None)) == sg.OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert _rotation(out.cpu().tolist()) is not None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sg.sgemm_topology_probe(out.data_ptr(), 256, sg._stream_handle(None))
    for _ in range(3):
        out.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert _rotation(out.cpu().tolist()) is not None
    assert _rotation(sg.topology(256)) is not None


def test_device_check_accepts_this_gpu(cuda_device):
    assert sg.sgemm_device_check(0) == sg.OK


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1536), (32, 2048, 1024), (128, 2048, 1536)])
def test_gemm_placement_claim_reports_a_duplicate_slot(cuda_device, M, K, N):
    """With SGEMM_F_CHECK_PLACEMENT the single GEMM checks that its workgroups
    covered every (XCD, slot) pair once.  A claim bit set in the workspace before the launch looks, to
    the workgroup that owns that pair, like a second workgroup on the same
    pair, whatever order the XCD's workgroups claim in: the launch reports
    SGEMM_ERR_TOPOLOGY instead of passing silently.  Its XCD's 32 arrivals
    still complete and clear the claim and arrival words, so the next launch
    is clean, and the output of a normal launch is unaffected."""
    x, w, X, W = gemm_inputs(M, K, N, 41, 42, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_CHECK_PLACEMENT)
    ws = g.new_workspace()
    Y = torch.empty((M, N), dtype=torch.float32, device=cuda_device)
    claim = ws[128:160].view(torch.int32)
    claim[3] = 1 << 5                       # XCD 3, slot 5 already claimed
    g(X, W, Y, ws)
    assert g.status(ws) == sg.ERR_TOPOLOGY
    assert int(claim.abs().sum()) == 0       # every XCD's claims were cleared by its last arrival
    assert int(ws[160:192].view(torch.int32).abs().sum()) == 0   # and so were the arrival counts
    g(X, W, Y, ws)
    assert g.status(ws) == sg.OK
    check(Y.cpu().numpy(), x, w)


def test_generator_on_device_matches_host(cuda_device):
    seed, a = synth.seed_for(2, 0, synth.T_WQ), synth.weight_scale(4096)
    ref = synth.uniform_bf16(seed, 33, 4096, a)
    t = synth.uniform_bf16_torch(seed, 33, 4096, a, cuda_device)
    assert np.array_equal(host_bits(t), ref)


SMALL = [(1, 1024, 1024), (1, 520, 1000), (2, 1032, 777), (3, 4104, 129), (7, 2056, 300),
         (8, 1024, 2048), (9, 776, 530), (15, 1032, 300), (16, 1024, 2048), (17, 776, 530),
         (31, 1000, 999), (33, 2048, 1536), (48, 520, 64), (64, 2048, 1536), (64, 8, 1), (1, 8, 1),
         (5, 8, 17), (13, 16, 3000), (40, 12288, 96)]


@pytest.mark.parametrize("M,K,N", SMALL)
def test_parity_small(cuda_device, M, K, N):
    x, w, X, W = gemm_inputs(M, K, N, 1000 + M, 2000 + K, cuda_device)
    g = sg.Gemm(M, K, N)
    Y = run(g, X, W).cpu().numpy()
    check(Y, x, w)


@pytest.mark.parametrize("M,K,N", [(1, 4096, 6144), (3, 4104, 129), (8, 1024, 2048), (13, 16, 3000),
                                   (1, 12288, 4096), (5, 8, 17), (16, 2048, 24576), (16, 1032, 3000),
                                   (16, 520, 1000)])
def test_round_robin_order_bitwise(cuda_device, M, K, N, monkeypatch):
    """The dot2 and MFMA paths' items round-robin over the XCD's streams (the
    default for one K split) or in contiguous ranges (SGEMM_DOT2_RR=0,
    SGEMM_MFMA_RR=0): the same products in the same order per output, so
    bitwise the same Y, and both within the bound."""
    x, w, X, W = gemm_inputs(M, K, N, 3000 + M, 4000 + K, cuda_device)
    out = {}
    for rr in ("1", "0"):
        monkeypatch.setenv("SGEMM_DOT2_RR", rr)
        monkeypatch.setenv("SGEMM_MFMA_RR", rr)
        g = sg.Gemm(M, K, N)
        st = g.describe()["stage"]
        assert st["path"] == ("dot2" if M < 16 else "mfma") and st["S"] == 1 and st["rr"] == int(rr), st
        out[rr] = run(g, X, W)
    assert torch.equal(out["1"], out["0"])
    check(out["1"].cpu().numpy(), x, w)


# One GPU's share of the Qwen3-8B decode projections under 8-way tensor parallelism:
# QKV and gate_up split by output columns (N / 8), O and down by K (K / 8).
TP8_SHARDS = [(4096, 768), (512, 4096), (4096, 3072), (1536, 4096)]


@pytest.mark.parametrize("M", [1, 16, 64])
@pytest.mark.parametrize("K,N", TP8_SHARDS)
def test_parity_tp8_shard_shapes(cuda_device, M, K, N):
    x, w, X, W = gemm_inputs(M, K, N, 5000 + M, 6000 + K + N, cuda_device)
    g = sg.Gemm(M, K, N)
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("M,K,N", SPLITK_SHAPES)
@pytest.mark.parametrize("splitk", [2, 5, 11])
def test_parity_forced_splitk(cuda_device, M, K, N, splitk):
    x, w, X, W = gemm_inputs(M, K, N, 3000 + M, 4000 + K, cuda_device)
    g = sg.Gemm(M, K, N, splitk=splitk)
    assert g.describe()["stage"]["S"] > 1
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("M", [1, 3, 8, 15])
def test_parity_mfma_path_for_small_m(cuda_device, M):
    K, N = 1032, 777
    x, w, X, W = gemm_inputs(M, K, N, 5000 + M, 6000, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_FORCE_MFMA)
    assert g.describe()["stage"]["path"] == "mfma"
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("waves,tn", [(4, 0), (8, 0), (8, 32), (4, 16)])
def test_parity_tilings(cuda_device, waves, tn):
    for M in (4, 24):
        K, N = 2048, 1040
        x, w, X, W = gemm_inputs(M, K, N, 7000 + M, 8000, cuda_device)
        path_tn = tn if M >= 16 else (tn // 4 if tn else 0)
        g = sg.Gemm(M, K, N, waves=waves, tn=path_tn)
        check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("M,K,N,ksl,splitk", KSL_CASES)
def test_parity_kslices(cuda_device, M, K, N, ksl, splitk):
    x, w, X, W = gemm_inputs(M, K, N, 9700 + M, 9800 + K, cuda_device)
    g = sg.Gemm(M, K, N, kslices=ksl, splitk=splitk)
    st = g.describe()["stage"]
    assert st["ksl"] == ksl and st["wpi"] == st["waves"]
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("M", [2, 20])
def test_bf16_output(cuda_device, M):
    K, N = 2056, 900
    x, w, X, W = gemm_inputs(M, K, N, 9000 + M, 9100, cuda_device)
    g = sg.Gemm(M, K, N, out_dtype=sg.OUT_BF16)
    y = run(g, X, W).float().cpu().numpy()
    check(y, x, w, bf16_out=True)


@pytest.mark.parametrize("flags", [sg.F_SYNC_AGENT, sg.F_W_CACHED, sg.F_W_SC1])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_sync_and_cache_variants_bitwise_equal(cuda_device, flags, M):
    K, N = 4096, 1536
    x, w, X, W = gemm_inputs(M, K, N, 9500 + M, 9600, cuda_device)
    S = 4 if M < 16 else 8
    base = run(sg.Gemm(M, K, N, splitk=S), X, W)
    other = run(sg.Gemm(M, K, N, splitk=S, flags=flags), X, W)
    assert torch.equal(base, other)
    check(base.cpu().numpy(), x, w)


@pytest.mark.parametrize("M,S", [(1, 1), (8, 4), (32, 8)])
def test_graph_replays_match_eager(cuda_device, M, S):
    """A HIP graph of sgemm_run (split-K counters included) replays to the
    eager result bitwise, with eager runs and host synchronisation between
    the replays."""
    K, N = 4096, 1536
    x, w, X, W = gemm_inputs(M, K, N, 9700 + M, 9800, cuda_device)
    g = sg.Gemm(M, K, N, splitk=S)
    ws = g.new_workspace()
    Ye = run(g, X, W, ws)
    Y = torch.empty_like(Ye)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g(X, W, Y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g(X, W, Y, ws)
    for r in range(4):
        Y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert g.status(ws) == sg.OK, r
        assert torch.equal(Y, Ye), r
        assert torch.equal(run(g, X, W, ws), Ye), r
    check(Ye.cpu().numpy(), x, w)


# ------------------------------------------------------------- exactness pins
def _int_inputs(M, K, N, dev):
    xb = synth.int_bf16(11, M, K, -3, 3)
    wb = synth.int_bf16(12, N, K, -3, 3)
    return xb, wb, device_tensor_bf16(xb, dev), device_tensor_bf16(wb, dev)


DECODE_SHAPES = [(1, 4096, 6144), (1, 4096, 4096), (1, 4096, 24576), (1, 12288, 4096),
                 (8, 12288, 4096), (16, 4096, 6144), (32, 4096, 24576), (64, 12288, 4096),
                 (1, 7168, 1536), (2, 7168, 18432), (4, 7168, 4096), (16, 7168, 1536)]


@pytest.mark.parametrize("M,K,N", DECODE_SHAPES)
def test_integer_inputs_bitwise_at_full_size(cuda_device, M, K, N):
    """Integer inputs in [-3, 3]: every partial sum is an integer below 2**24,
    so fp32 accumulation is exact in any order (split-K included) and every
    output element must equal the exact product bitwise."""
    xb, wb, X, W = _int_inputs(M, K, N, cuda_device)
    Y = run(sg.Gemm(M, K, N), X, W).cpu().numpy()
    xi = synth.bf16_bits_to_f32(xb).astype(np.float64)
    wi = synth.bf16_bits_to_f32(wb).astype(np.float64)
    ref = (xi @ wi.T).astype(np.float32)       # exact: integers below 2**53 in float64
    assert np.array_equal(Y, ref)


@pytest.mark.parametrize("M,K,N", [(1, 1024, 1024), (8, 7168, 4096), (64, 12288, 4096), (3, 4096, 24576)])
def test_all_ones_gives_K(cuda_device, M, K, N):
    X = torch.ones((M, K), dtype=torch.bfloat16, device=cuda_device)
    W = torch.ones((N, K), dtype=torch.bfloat16, device=cuda_device)
    Y = run(sg.Gemm(M, K, N), X, W)
    assert bool(torch.all(Y == float(K)))


@pytest.mark.parametrize("M", [1, 5, 16, 64])
def test_one_hot_weights_copy_columns(cuda_device, M):
    K, N = 4096, 2048
    perm = np.random.default_rng(M).permutation(K)[:N]
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=cuda_device)
    W[torch.arange(N, device=cuda_device), torch.from_numpy(perm).to(cuda_device)] = 1.0
    xb = synth.normal_bf16(77 + M, M, K)
    X = device_tensor_bf16(xb, cuda_device)
    Y = run(sg.Gemm(M, K, N), X, W).cpu().numpy()
    assert np.array_equal(Y, synth.bf16_bits_to_f32(xb)[:, perm])


@pytest.mark.parametrize("M", [1, 8, 24, 64])
def test_power_of_two_scaling_and_determinism(cuda_device, M):
    K, N = 7168, 4096
    x, w, X, W = gemm_inputs(M, K, N, 31 + M, 32, cuda_device, w_on_device=True)
    g = sg.Gemm(M, K, N)
    ws = g.new_workspace()
    Y1 = run(g, X, W, ws)
    Y2 = run(g, X, W, ws)
    assert torch.equal(Y1, Y2)
    Y3 = run(g, X * 32.0, W * 0.125, ws)
    assert torch.equal(Y3, Y1 * 4.0)


# ----------------------------------------------------------- full-size workloads
def test_single_gemm_1x1024x1024(cuda_device):
    """The 1 x 1024 x 1024 GEMM (fp32 output), every element."""
    _full_size(cuda_device, 1, 1024, 1024, workload=1)


@pytest.mark.parametrize("M,K,N", [(1, 4096, 6144), (1, 4096, 4096), (1, 4096, 24576), (1, 12288, 4096)])
def test_decode_projections_m1_full_size(cuda_device, M, K, N):
    _full_size(cuda_device, M, K, N, workload=2)


@pytest.mark.parametrize("M", [8, 16, 32, 64])
@pytest.mark.parametrize("K,N", [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)])
def test_decode_projections_m8_to_64_full_size(cuda_device, M, K, N):
    _full_size(cuda_device, M, K, N, workload=3)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("N", [1536, 4096, 18432])
def test_k7168_decode_gemms_full_size(cuda_device, M, N):
    _full_size(cuda_device, M, 7168, N, workload=4)


def _full_size(dev, M, K, N, workload):
    """Every output element against the oracle, on the configuration's seeded
    inputs (weights drawn on the device by the counter-based generator, checked
    row-wise against the host generator), in the plan the bench uses."""
    seed_x = synth.seed_for(workload, 0, synth.T_X, M)
    seed_w = synth.seed_for(workload, 0, synth.T_WQ, K % 251 + N % 241)
    x, _, X, W = gemm_inputs(M, K, N, seed_x, seed_w, dev, w_on_device=True)
    Y = run(sg.Gemm(M, K, N), X, W).cpu().numpy()
    w = device_weights_checked(W, seed_w, K)
    ratio = check(Y, x, w)
    report("gemm %dx%dx%d" % (M, K, N), ratio, workload=workload)


@pytest.mark.parametrize("n16", [1, 63, 64, 777, 12345, 1 << 20, (50 << 20) // 16 + 5])
@pytest.mark.parametrize("pattern,grid", [(0, 256), (1, 256), (1, 8), (0, 1024)])
def test_read_probe_reads_every_byte_once(cuda_device, n16, pattern, grid):
    """The attainable-bandwidth probe xors every 32-bit word it reads into the
    sink: equal to the host xor of the buffer only if each word was read
    exactly once (a missed or repeated chunk changes it for random data)."""
    rng = np.random.default_rng(n16 * 7 + pattern)
    host = rng.integers(0, 2 ** 32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(cuda_device)
    sink = sg.read_probe(buf, pattern, grid=grid)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host))


@pytest.mark.parametrize("M,K,N,splitk", MTI_CASES)
def test_parity_mtile_items(cuda_device, M, K, N, splitk):
    """The m-tile-item ablation (one 16-row m-tile per item, neighbouring waves
    share a column block's weights through the caches) computes the same
    GEMM."""
    x, w, X, W = gemm_inputs(M, K, N, 9900 + M, 9950 + K, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_MTILE_ITEMS, splitk=splitk)
    st = g.describe()["stage"]
    assert st["mtiles"] == -(-M // 16) and st["ta"] == 1
    check(run(g, X, W).cpu().numpy(), x, w)


# ----------------------------------------------------- K-chunked MFMA path
KC_SMALL = [(16, 1024, 2048, 0, 0), (17, 776, 530, 2, 0), (33, 2048, 1536, 4, 0), (48, 520, 64, 6, 0),
            (64, 2048, 1536, 6, 0), (64, 1000, 1000, 4, 3), (5, 1032, 777, 2, 0), (64, 8, 1, 2, 0),
            (32, 3000, 700, 8, 2), (20, 12288, 300, 4, 5), (64, 4104, 129, 6, 2), (1, 1024, 1024, 8, 0),
            (64, 4096, 1536, 3, 0), (40, 2056, 900, 3, 2)]


@pytest.mark.parametrize("M,K,N,ntw,splitk", KC_SMALL)
def test_parity_kchunk_small(cuda_device, M, K, N, ntw, splitk):
    """The K-chunked MFMA path (eight waves on one block of tiles, X double-
    buffered through LDS in 512-wide K chunks): ragged M, K and N, forced tile
    counts and split counts, every output element."""
    x, w, X, W = gemm_inputs(M, K, N, 8100 + M, 8200 + K, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_KCHUNK, tn=16 * ntw, splitk=splitk)
    st = g.describe()["stage"]
    assert st["path"] == "kc" and (ntw == 0 or st["tb"] == ntw)
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("M", [16, 32, 64])
@pytest.mark.parametrize("K,N", [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)])
def test_kchunk_decode_projections_full_size(cuda_device, M, K, N):
    """The decode projections at M = 16, 32, 64 on the K-chunked path, every
    output element against the oracle."""
    seed_x = synth.seed_for(3, 0, synth.T_X, M)
    seed_w = synth.seed_for(3, 0, synth.T_WQ, K % 251 + N % 241)
    x, _, X, W = gemm_inputs(M, K, N, seed_x, seed_w, cuda_device, w_on_device=True)
    g = sg.Gemm(M, K, N, flags=sg.F_KCHUNK)
    assert g.describe()["stage"]["path"] == "kc"
    Y = run(g, X, W).cpu().numpy()
    w = device_weights_checked(W, seed_w, K)
    report("kc gemm %dx%dx%d" % (M, K, N), check(Y, x, w), workload=3)


@pytest.mark.parametrize("M,K,N,splitk", [(64, 4096, 24576, 0), (64, 12288, 4096, 2), (17, 7168, 1536, 3),
                                          (48, 4096, 4096, 4)])
def test_kchunk_integer_inputs_bitwise(cuda_device, M, K, N, splitk):
    """Integer inputs: every partial sum is exact in fp32, so the K-chunked
    path (eight-wave tree reduction, split-K partials) must equal the exact
    product bitwise."""
    xb, wb, X, W = _int_inputs(M, K, N, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_KCHUNK, splitk=splitk)
    Y = run(g, X, W).cpu().numpy()
    ref = (synth.bf16_bits_to_f32(xb).astype(np.float64) @ synth.bf16_bits_to_f32(wb).astype(np.float64).T)
    assert np.array_equal(Y, ref.astype(np.float32))


@pytest.mark.parametrize("splitk", [1, 3])
def test_kchunk_graph_replays_and_repeat(cuda_device, splitk):
    """Repeated eager runs and HIP graph replays of the K-chunked path give
    bitwise the same output (split-K counters reset by their owners)."""
    M, K, N = 40, 4096, 2048
    x, w, X, W = gemm_inputs(M, K, N, 8300, 8400, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_KCHUNK, splitk=splitk)
    ws = g.new_workspace()
    Ye = run(g, X, W, ws)
    assert torch.equal(run(g, X, W, ws), Ye)
    Y = torch.empty_like(Ye)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g(X, W, Y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g(X, W, Y, ws)
    for r in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert g.status(ws) == sg.OK, r
        assert torch.equal(Y, Ye), r
    check(Ye.cpu().numpy(), x, w)


@pytest.mark.parametrize("M,K,N", [(64, 4096, 1536), (48, 2056, 900), (33, 776, 530), (64, 12288, 300)])
@pytest.mark.parametrize("tm,msplit", [(32, False), (64, False), (16, True), (32, True)])
def test_parity_mtile_windows_and_msplit(cuda_device, M, K, N, tm, msplit):
    """The M-major window ablation with 32- and 64-row windows, and the
    M-split order (column block fastest), compute the same GEMM."""
    x, w, X, W = gemm_inputs(M, K, N, 9960 + M, 9970 + K, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_MSPLIT if msplit else sg.F_MTILE_ITEMS, tm=tm)
    st = g.describe()["stage"]
    assert st["mtiles"] == -(-M // tm) and st["nfast"] == int(msplit)
    check(run(g, X, W).cpu().numpy(), x, w)


def _random_default_cases(n=40, seed=20261205):
    """Seeded random shapes for the planner's default plans: M in 1..256 (so
    every path is drawn: dot2, MFMA, K-chunked, large tiles), K a multiple
    of 8 up to 12288, N up to 6000, fp32 or bf16 output."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 16)), int(rng.integers(16, 65)), int(rng.integers(65, 257))]))
        K = int(rng.integers(1, 1537)) * 8
        N = int(rng.integers(1, 6001))
        out.append((M, K, N, int(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("M,K,N,bf16", _random_default_cases())
def test_random_shapes_default_plans(cuda_device, M, K, N, bf16):
    """Default plans on seeded random shapes, every element against the
    oracle (bf16 outputs within one more bf16 ulp)."""
    x, w, X, W = gemm_inputs(M, K, N, 14000 + M, 14100 + K % 1000, cuda_device)
    g = sg.Gemm(M, K, N, out_dtype=sg.OUT_BF16 if bf16 else sg.OUT_F32)
    Y = run(g, X, W).float().cpu().numpy()
    check(Y, x, w, bf16_out=bool(bf16))


@pytest.mark.parametrize("M,K,N,S", [(17, 4096, 4096, 4), (32, 4096, 2048, 4), (36, 4096, 2048, 4), (48, 4096, 3000, 4),
                                     (10, 7168, 3072, 2), (12, 7168, 4096, 2), (15, 6144, 4096, 2), (15, 8192, 3500, 2)])
def test_measured_split_rule_plans(cuda_device, M, K, N, S):
    """The planner's measured split rules (four K splits at M = 17-48 on
    4096-deep narrow outputs; two for dot2 at M = 10-15, K = 6144-8192):
    the plan takes them, and every output element matches the oracle."""
    g = sg.Gemm(M, K, N)
    assert g.describe()["stage"]["S"] == S
    x, w, X, W = gemm_inputs(M, K, N, 15000 + M, 15100 + N % 1000, cuda_device)
    check(run(g, X, W).cpu().numpy(), x, w)
