"""rmm_matmul_noalloc (the call that allocates nothing) against rmm_matmul.

Through the C ABI: the same operands go to rmm_matmul (caller workspace)
and to rmm_matmul_noalloc (the library's per-GPU scratch array); index sets
and products must be bit-identical, on consecutive calls where a later one is
smaller than the one before (the array keeps the last call's contents), and
a call that needs more scratch than the array holds is refused before it
writes anything.
"""

import numpy as np
import pytest
import torch

import synth
from input_adaptive_reduced_colnorm_amd import rmm
from oracle import rmm_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    rmm.lib()
    return torch.device("cuda:0")


def _both(A, B, rho, dev):
    L = rmm.lib()
    n, d = A.shape
    m = B.shape[1]
    k = rmm.k(rho, d)
    sh = torch.cuda.current_stream(dev).cuda_stream
    idx1 = torch.full((k,), -7, dtype=torch.int32, device=dev)
    Y1 = torch.full((n, m), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, L.rmm_matmul_workspace(n, d, m, d, rmm.RMM_BF16, rho)), dtype=torch.uint8, device=dev)
    st = L.rmm_matmul(A.data_ptr(), B.data_ptr(), rmm.RMM_BF16, n, d, m, d, m, rho, idx1.data_ptr(), Y1.data_ptr(),
                      rmm.RMM_FP32, m, ws.data_ptr(), ws.numel(), sh)
    assert st == 0, rmm.status_str(st)
    idx2 = torch.full((k,), -7, dtype=torch.int32, device=dev)
    Y2 = torch.full((n, m), float("nan"), dtype=torch.float32, device=dev)
    st = L.rmm_matmul_noalloc(A.data_ptr(), B.data_ptr(), rmm.RMM_BF16, n, d, m, d, m, rho, idx2.data_ptr(),
                              Y2.data_ptr(), rmm.RMM_FP32, m, sh)
    assert st == 0, rmm.status_str(st)
    torch.cuda.synchronize()
    return idx1, Y1, idx2, Y2


def test_noalloc_matches_the_workspace_call(dev):
    cases = [
        (synth.mlp_down(n=1024, d=4096, m=512, rhos=(0.7,)), 0.7),   # packed prefill, ~6 MB of scratch
        (synth.mlp_down(n=300, d=1000, m=264, rhos=(0.5,)), 0.5),    # smaller, ragged tiles
        (synth.decode_qkv(), 0.8),                                    # decode GEMV, slice partials
        (synth.decode_qkv(n=5, d=1024, m=776), 0.8),                  # smaller decode
        (synth.mlp_down(n=300, d=1000, m=264, rhos=(0.5,)), 1.0),    # dense: no scratch at all
    ]
    for w, rho in cases:
        A, B = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
        print(f"noalloc {tuple(A.shape)} x {tuple(B.shape)} rho={rho}", flush=True)
        idx1, Y1, idx2, Y2 = _both(A, B, rho, dev)
        assert torch.equal(idx1, idx2)
        assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
        idx_o, _ = O.matmul(w.tensors["A"].float().numpy(), w.tensors["B"].float().numpy(), rho,
                            rows=np.arange(1))
        np.testing.assert_array_equal(idx2.cpu().numpy(), idx_o)


def test_noalloc_refuses_a_call_beyond_its_scratch(dev):
    # n x ceil(0.9 d) bf16 packed A alone is 2 * 4096 * 12928 bytes > 32 MiB
    L = rmm.lib()
    n, d, m = 4096, 14336, 256
    A = torch.zeros((n, d), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((d, m), dtype=torch.bfloat16, device=dev)
    k = rmm.k(0.9, d)
    idx = torch.full((k,), -7, dtype=torch.int32, device=dev)
    Y = torch.full((n, m), 3.0, dtype=torch.float32, device=dev)
    st = L.rmm_matmul_noalloc(A.data_ptr(), B.data_ptr(), rmm.RMM_BF16, n, d, m, d, m, 0.9, idx.data_ptr(),
                              Y.data_ptr(), rmm.RMM_FP32, m, torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert st == 6, rmm.status_str(st)   # RMM_ERR_WORKSPACE
    assert bool((idx == -7).all()) and bool((Y == 3.0).all())
