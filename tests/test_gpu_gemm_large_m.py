"""GPU parity of the single GEMM beyond 64 rows (M = 65..256).

Those shapes run on the large-tile MFMA path by default (four waves over a
workgroup tile of up to 256 rows, X and W fragments staged in LDS) and, with
SGEMM_F_KCHUNK, on the K-chunked MFMA path in 64-row m-blocks.  In both the
m-blocks of a column block are neighbouring items that an XCD's workgroups
take round-robin (so they share the block's weights through that XCD's L2).
Every output element is compared with the CPU oracle: ragged M, K and N that span
several m-blocks, column blocks and splits, forced tile and split counts,
bf16 output, integer inputs (bitwise), run-to-run and graph-replay
determinism, and the decode projection shapes at M = 128 and 256 at full
size.  Every call goes through the C ABI (ctypes) into libsgemm.so.
"""
import numpy as np
import pytest

import chiplet_aware_persistent_amd as sg
import synth
from helpers import check, device_tensor_bf16, device_weights_checked, gemm_inputs, report

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run(g, X, W, ws=None):
    Y = torch.empty((g.M, g.N), dtype=torch.float32 if g.out_dtype == sg.OUT_F32 else torch.bfloat16,
                    device=X.device)
    if ws is None:
        ws = g.new_workspace()
    g(X, W, Y, ws)
    rc = g.status(ws)
    assert rc == sg.OK, sg.status_string(rc)
    return Y


def _plan_checks(g, M):
    st = g.describe()["stage"]
    if st["path"] == "kc":
        assert st["ta"] == 4 and st["mb"] == -(-M // 64) and st["rr"] == 1, st
    else:
        assert st["path"] == "lt" and st["mb"] == -(-M // (32 * st["ta"])) and st["rr"] == 1, st
    return st


# Beyond 64 rows the default plan is the large-tile path; SGEMM_F_KCHUNK
# takes the K-chunked path in 64-row m-blocks.
PATHS = [("lt", 0), ("kc", sg.F_KCHUNK)]


LARGE_SMALL = [(65, 1032, 777, 0, 0), (65, 1032, 777, 2, 3), (80, 520, 64, 0, 0), (100, 2048, 1536, 4, 0),
               (100, 2048, 1536, 6, 2), (128, 1024, 4096, 0, 0), (129, 4104, 129, 3, 2), (144, 776, 530, 2, 0),
               (200, 3000, 700, 0, 0), (200, 3000, 700, 4, 3), (255, 2056, 900, 6, 0), (256, 4096, 1024, 0, 0),
               (256, 4096, 1024, 2, 4), (256, 8, 1, 0, 0), (192, 12288, 300, 0, 5)]


@pytest.mark.parametrize("M,K,N,ntw,splitk", LARGE_SMALL)
def test_parity_large_m_small(cuda_device, M, K, N, ntw, splitk):
    """K-chunked path in 64-row m-blocks, forced tile counts and splits."""
    x, w, X, W = gemm_inputs(M, K, N, 12100 + M, 12200 + K, cuda_device)
    g = sg.Gemm(M, K, N, flags=sg.F_KCHUNK, tn=16 * ntw, splitk=splitk)
    st = _plan_checks(g, M)
    assert st["path"] == "kc"
    assert ntw == 0 or st["tb"] == ntw
    # forced splits are whole chunk groups, so a short K may take fewer
    assert splitk == 0 or 1 <= st["S"] <= splitk
    check(run(g, X, W).cpu().numpy(), x, w)


LT_SMALL = [(65, 1032, 777, 0, 0), (65, 1032, 777, 96, 3), (80, 520, 64, 0, 0), (100, 2048, 1536, 192, 0),
            (100, 2048, 1536, 96, 2), (128, 1024, 4096, 0, 0), (129, 4104, 129, 96, 2), (144, 776, 530, 192, 0),
            (200, 3000, 700, 0, 0), (200, 3000, 700, 96, 3), (255, 2056, 900, 192, 0), (256, 4096, 1024, 0, 0),
            (256, 4096, 1024, 96, 4), (256, 8, 1, 0, 0), (192, 12288, 300, 0, 5), (96, 4104, 777, 192, 7)]


LT8_SMALL = [(65, 1032, 777, 192, 0, 0), (100, 2048, 1536, 384, 128, 2), (129, 4104, 129, 192, 256, 2),
             (200, 3000, 700, 192, 256, 3), (256, 4096, 1024, 384, 128, 0), (256, 8, 1, 192, 64, 0),
             (144, 776, 530, 384, 0, 0), (192, 12288, 300, 192, 0, 5)]


@pytest.mark.parametrize("M,K,N,tn,tm,splitk", LT8_SMALL)
def test_parity_large_tile_eight_waves(cuda_device, M, K, N, tn, tm, splitk):
    """Large-tile path with eight waves (2 x 4 over tiles of 192 or 384
    columns): ragged shapes, forced tile sizes and splits."""
    x, w, X, W = gemm_inputs(M, K, N, 12900 + M, 13000 + K, cuda_device)
    g = sg.Gemm(M, K, N, waves=8, tn=tn, tm=tm, splitk=splitk)
    st = _plan_checks(g, M)
    assert st["path"] == "lt" and st["waves"] == 8 and st["CB"] == tn and (tm == 0 or 32 * st["ta"] == tm)
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("M,K,N,tn,splitk", LT_SMALL)
def test_parity_large_tile_small(cuda_device, M, K, N, tn, splitk):
    """Large-tile path, four waves: ragged M, K and N, forced tile widths (96
    or 192 columns) and split counts, every element against the oracle."""
    x, w, X, W = gemm_inputs(M, K, N, 12700 + M, 12800 + K, cuda_device)
    g = sg.Gemm(M, K, N, waves=4, tn=tn, splitk=splitk)
    st = _plan_checks(g, M)
    assert st["path"] == "lt"
    assert tn == 0 or st["CB"] == tn
    assert splitk == 0 or 1 <= st["S"] <= splitk
    check(run(g, X, W).cpu().numpy(), x, w)


@pytest.mark.parametrize("path,flags", PATHS)
@pytest.mark.parametrize("M", [65, 130])
def test_large_m_bf16_output(cuda_device, M, path, flags):
    K, N = 2056, 1000
    x, w, X, W = gemm_inputs(M, K, N, 12300 + M, 12301, cuda_device)
    g = sg.Gemm(M, K, N, out_dtype=sg.OUT_BF16, flags=flags)
    assert _plan_checks(g, M)["path"] == path
    Y = run(g, X, W).float().cpu().numpy()
    check(Y, x, w, bf16_out=True)


@pytest.mark.parametrize("path,flags", PATHS)
@pytest.mark.parametrize("M,K,N,splitk", [(128, 4096, 24576, 0), (256, 12288, 4096, 0), (192, 4096, 6144, 2),
                                          (97, 7168, 18432, 0)])
def test_large_m_integer_inputs_bitwise(cuda_device, M, K, N, splitk, path, flags):
    """Integer inputs in [-3, 3]: every partial sum is an integer below 2**24,
    exact in fp32 in any order, so every element equals the exact product."""
    xb = synth.int_bf16(11, M, K, -3, 3)
    wb = synth.int_bf16(12, N, K, -3, 3)
    X, W = device_tensor_bf16(xb, cuda_device), device_tensor_bf16(wb, cuda_device)
    g = sg.Gemm(M, K, N, splitk=splitk, flags=flags)
    assert _plan_checks(g, M)["path"] == path
    Y = run(g, X, W).cpu().numpy()
    ref = synth.bf16_bits_to_f32(xb).astype(np.float64) @ synth.bf16_bits_to_f32(wb).astype(np.float64).T
    assert np.array_equal(Y, ref.astype(np.float32))


@pytest.mark.parametrize("path,flags", PATHS)
@pytest.mark.parametrize("splitk", [1, 3])
def test_large_m_repeat_and_graph_replays(cuda_device, splitk, path, flags):
    """Repeated eager runs and replays of a captured HIP graph give bitwise
    the same output (split-K counters reset by their owners)."""
    M, K, N = 200, 4096, 2048
    x, w, X, W = gemm_inputs(M, K, N, 12400, 12401, cuda_device)
    g = sg.Gemm(M, K, N, splitk=splitk, flags=flags)
    assert _plan_checks(g, M)["path"] == path
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


@pytest.mark.parametrize("path,flags", PATHS)
@pytest.mark.parametrize("M", [128, 256])
@pytest.mark.parametrize("K,N", [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)])
def test_decode_projections_m128_m256_full_size(cuda_device, M, K, N, path, flags):
    """The four projection shapes at M = 128 and 256, every output element
    against the oracle, in the plan the bench's large-M lines use."""
    seed_x = synth.seed_for(3, 0, synth.T_X, M)
    seed_w = synth.seed_for(3, 0, synth.T_WQ, K % 251 + N % 241)
    x, _, X, W = gemm_inputs(M, K, N, seed_x, seed_w, cuda_device, w_on_device=True)
    g = sg.Gemm(M, K, N, flags=flags)
    assert _plan_checks(g, M)["path"] == path
    Y = run(g, X, W).cpu().numpy()
    w = device_weights_checked(W, seed_w, K)
    report("gemm %s %dx%dx%d" % (path, M, K, N), check(Y, x, w), workload="large_m")


def _random_large_tile_cases(n=24, seed=20261204):
    """Seeded random shapes and large-tile plans: M in 49..256, K a multiple
    of 8 up to 8200 (ragged against the 64-wide steps), N up to 5000, the
    tile (waves, rows, columns) and the split count drawn from what is
    built."""
    rng = np.random.default_rng(seed)
    tiles = [(4, 64, 96), (4, 128, 96), (4, 128, 192), (4, 256, 96), (8, 64, 192), (8, 128, 192),
             (8, 128, 384), (8, 256, 192)]
    out = []
    for _ in range(n):
        M = int(rng.integers(49, 257))
        K = int(rng.integers(1, 1026)) * 8
        N = int(rng.integers(1, 5001))
        w, tm, tn = tiles[int(rng.integers(len(tiles)))]
        S = int(rng.choice([0, 0, 1, 2, 3, 5, 8]))
        out.append((M, K, N, w, tm, tn, S))
    return out


@pytest.mark.parametrize("M,K,N,waves,tm,tn,splitk", _random_large_tile_cases())
def test_large_tile_random_shapes(cuda_device, M, K, N, waves, tm, tn, splitk):
    """Seeded random shapes on forced large-tile plans (M = 49..64 included,
    where the path is forced through the tile arguments), every element
    against the oracle."""
    x, w, X, W = gemm_inputs(M, K, N, 13100 + M + K % 97, 13200 + N, cuda_device)
    import os
    old = os.environ.get("SGEMM_LT_MIN_M")
    os.environ["SGEMM_LT_MIN_M"] = "49"
    try:
        g = sg.Gemm(M, K, N, waves=waves, tm=tm, tn=tn, splitk=splitk)
    finally:
        if old is None:
            del os.environ["SGEMM_LT_MIN_M"]
        else:
            os.environ["SGEMM_LT_MIN_M"] = old
    st = g.describe()["stage"]
    assert st["path"] == "lt" and st["waves"] == waves and 32 * st["ta"] == tm and st["CB"] == tn
    check(run(g, X, W).cpu().numpy(), x, w)
