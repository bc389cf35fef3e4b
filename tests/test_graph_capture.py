"""The hot path captured once in a HIP graph and replayed.

Each operation runs eagerly into caller-owned outputs, is then captured with
the same outputs and workspace, and the graph is replayed several times.
Between replays the program clears the outputs and runs other eager work (the
same operation on other operands, into other buffers).  The kernels sum in a
fixed order and the library makes no allocating or synchronous HIP call, so
every replay must equal the eager call bitwise.
"""

import pytest
import torch

import synth
from input_adaptive_reduced_colnorm_amd import rmm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    rmm.lib()
    return torch.device("cuda:0")


def _clear(outs):
    for o in outs:
        if o.is_floating_point():
            o.fill_(float("nan"))
        else:
            o.fill_(-7)


def _capture_and_replay(dev, what, run, outs, other, replays=4):
    """run(): the operation into the tensors `outs` (captured); other(): eager
    work between replays."""
    print(f"graph {what}: eager", flush=True)
    _clear(outs)
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    print(f"graph {what}: capture", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(replays):
        _clear(outs)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"{what}: replay {r}, output {i} differs from the eager call"
    print(f"graph {what}: {replays} replays equal", flush=True)
    del g


def _linear_case(dev, w, rho, other_w):
    A, B = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
    n, d = A.shape
    m = B.shape[1]
    idx = torch.empty(rmm.k(rho, d), dtype=torch.int32, device=dev)
    Y = torch.empty((n, m), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, rmm.matmul_workspace(n, d, m, d, A.dtype, rho)), dtype=torch.uint8, device=dev)
    A2, B2 = other_w.tensors["A"].to(dev), other_w.tensors["B"].to(dev)

    def run():
        rmm.matmul(A, B, rho, workspace=ws, out=Y, idx=idx)

    def other():
        rmm.matmul(A2, B2, 0.5)

    return run, [idx, Y], other


@pytest.mark.parametrize("case", ["prefill", "prefill_last_wave", "decode"])
def test_matmul_graph_replays(dev, case):
    # prefill: column energies, the select + gather launch and the GEMM;
    # prefill_last_wave: the GEMM as two launches (whole waves of 256 x 256
    # tiles, then a 128 x 128 column band); decode: the ranking GEMV and the
    # ordered sum of its slices
    other = synth.mlp_down(n=300, d=1000, m=264, rhos=(0.5,))
    if case == "prefill":
        run, outs, oth = _linear_case(dev, synth.mlp_down(n=1024, d=4096, m=512, rhos=(0.7,)), 0.7, other)
    elif case == "prefill_last_wave":
        run, outs, oth = _linear_case(dev, synth.mlp_down(n=500, d=448, m=34776, rhos=(0.5,)), 0.5, other)
    else:
        run, outs, oth = _linear_case(dev, synth.decode_qkv(), 0.8, other)
    _capture_and_replay(dev, case, run, outs, oth)


def test_noalloc_graph_replays(dev):
    # the call that allocates nothing, on the library's own scratch array
    w = synth.mlp_down(n=1024, d=4096, m=512, rhos=(0.7,))
    A, B = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
    n, d = A.shape
    m = B.shape[1]
    rho = 0.7
    L = rmm.lib()
    idx = torch.empty(rmm.k(rho, d), dtype=torch.int32, device=dev)
    Y = torch.empty((n, m), dtype=torch.float32, device=dev)
    o = synth.mlp_down(n=300, d=1000, m=264, rhos=(0.5,))
    A2, B2 = o.tensors["A"].to(dev), o.tensors["B"].to(dev)

    def run():
        st = L.rmm_matmul_noalloc(A.data_ptr(), B.data_ptr(), rmm.RMM_BF16, n, d, m, d, m, rho, idx.data_ptr(),
                                  Y.data_ptr(), rmm.RMM_FP32, m, torch.cuda.current_stream(dev).cuda_stream)
        assert st == 0, rmm.status_str(st)

    def other():
        rmm.matmul(A2, B2, 0.5)

    _capture_and_replay(dev, "noalloc", run, [idx, Y], other)


def test_attention_graph_replays(dev):
    # QK^T scores over 800 tiles (the persistent score kernel), PV over fp32 P
    # in place (scoring, then the product split into contraction ranges and
    # their ordered sum), and a decode attention step (the streaming QK pass,
    # softmax with the key ranking, PV over the kept lists)
    wq = synth.gqa_qk(hq=32, hkv=8, t=1100, dh=128, rho=0.5)
    Q, K = wq.tensors["Q"].to(dev), wq.tensors["K"].to(dev)
    idx_q = torch.empty((32, rmm.k(0.5, 128)), dtype=torch.int32, device=dev)
    S = torch.empty((32, 1100, 1100), dtype=torch.float32, device=dev)
    ws_q = torch.empty(max(1, rmm.qk_workspace(32, 1100, 1100, 128, Q.dtype, 0.5)), dtype=torch.uint8, device=dev)
    wo = synth.gqa_qk(hq=8, hkv=2, t=300, dh=128, rho=0.5)
    Q2, K2 = wo.tensors["Q"].to(dev), wo.tensors["K"].to(dev)
    _capture_and_replay(dev, "qk", lambda: rmm.qk(Q, K, 0.5, workspace=ws_q, out=S, idx=idx_q), [idx_q, S],
                        lambda: rmm.qk(Q2, K2, 0.5))
    del S

    wp = synth.attn_pv(h=4, hkv=2, tq=96, tk=1024, dv=64, rho=0.5)
    P, V = wp.tensors["P"].to(dev), wp.tensors["V"].to(dev)
    idx_p = torch.empty((4, rmm.k(0.5, 1024)), dtype=torch.int32, device=dev)
    Ob = torch.empty((4, 96, 64), dtype=torch.float32, device=dev)
    ws_p = torch.empty(max(1, rmm.pv_workspace(4, 96, 1024, 64, P.dtype, V.dtype, 0.5)), dtype=torch.uint8,
                       device=dev)
    _capture_and_replay(dev, "pv", lambda: rmm.pv(P, V, 0.5, workspace=ws_p, out=Ob, idx=idx_p), [idx_p, Ob],
                        lambda: rmm.pv(P[:2], V[:1], 0.2))

    wd = synth.decode_attn_qk(hq=32, hkv=8, tq=1, tk=8192, dh=128)
    Qd, Kd = wd.tensors["Q"].to(dev), wd.tensors["K"].to(dev)
    wl = synth.attn_pv(h=32, hkv=8, tq=1, tk=8192, dv=128, rho=0.5, with_logits=True)
    Ld, Vd = wl.tensors["L"].to(dev), wl.tensors["V"].to(dev)
    k_att = rmm.k(0.5, 8192)
    idx_d = torch.empty((32, rmm.k(0.5, 128)), dtype=torch.int32, device=dev)
    Sd = torch.empty((32, 1, 8192), dtype=torch.float32, device=dev)
    Pd = torch.empty((32, 1, 8192), dtype=torch.float32, device=dev)
    Ed = torch.empty((32, 8192), dtype=torch.float32, device=dev)
    idx_k = torch.empty((32, k_att), dtype=torch.int32, device=dev)
    Od = torch.empty((32, 1, 128), dtype=torch.float32, device=dev)

    def step():
        rmm.qk(Qd, Kd, 0.5, out=Sd, idx=idx_d)
        rmm.softmax_select(Ld, 0.5, P=Pd, energy=Ed, idx=idx_k)
        rmm.pv_idx(Pd, Vd, idx_k, out=Od)

    _capture_and_replay(dev, "decode attention", step, [idx_d, Sd, Pd, Ed, idx_k, Od],
                        lambda: rmm.qk(Q2, K2, 0.5))
