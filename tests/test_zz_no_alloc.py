"""sgemm_run_noalloc (the single GEMM over the library's own static device
array, for callers that cannot allocate) against sgemm_run with a caller
workspace: bitwise the same output on two calls in a row, the second with a
smaller input, through the C ABI."""
import numpy as np
import pytest

import chiplet_aware_persistent_amd as sg
from helpers import check, gemm_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _with_workspace(g, X, W):
    Y = torch.empty((g.M, g.N), dtype=torch.float32, device=X.device)
    ws = g.new_workspace()
    g(X, W, Y, ws)
    assert g.status(ws) == sg.OK
    return Y


def _no_alloc(g, X, W):
    Y = torch.full((g.M, g.N), float("nan"), dtype=torch.float32, device=X.device)
    rc = sg.sgemm_run_noalloc(g.handle, X.data_ptr(), W.data_ptr(), Y.data_ptr(),
                              int(torch.cuda.current_stream().cuda_stream))
    assert rc == sg.OK, sg.status_string(rc)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("first,second", [((64, 4096, 24576, 4), (16, 2048, 3000, 3)),
                                          ((32, 12288, 4096, 8), (3, 1032, 777, 2)),
                                          ((64, 7168, 4096, 0), (1, 1024, 1024, 0)),
                                          ((200, 4096, 6144, 3), (128, 2048, 1536, 0)),
                                          ((256, 4096, 6144, 0), (96, 4096, 4096, 0))])
def test_no_alloc_matches_workspace_run_twice(cuda_device, first, second):
    for i, (M, K, N, S) in enumerate((first, second)):
        x, w, X, W = gemm_inputs(M, K, N, 700 + i, 800 + K, cuda_device)
        g = sg.Gemm(M, K, N, splitk=S)
        ref = _with_workspace(g, X, W)
        got = _no_alloc(g, X, W)
        assert torch.equal(got, ref), (M, K, N, S)
        check(got.cpu().numpy(), x, w)


def test_no_alloc_refuses_oversize_and_check_plans(cuda_device):
    X = torch.zeros(16, dtype=torch.bfloat16, device=cuda_device)
    g = sg.Gemm(64, 4096, 24576, splitk=16)          # 96 MiB of partials
    assert sg.sgemm_run_noalloc(g.handle, X.data_ptr(), X.data_ptr(), X.data_ptr(), 0) == sg.ERR_WORKSPACE
    g2 = sg.Gemm(4, 1024, 1024, flags=sg.F_CHECK_PLACEMENT)
    assert sg.sgemm_run_noalloc(g2.handle, X.data_ptr(), X.data_ptr(), X.data_ptr(), 0) == sg.ERR_UNSUPPORTED
    assert sg.sgemm_run_noalloc(g2.handle, 0, X.data_ptr(), X.data_ptr(), 0) == sg.ERR_INVALID_ARG
