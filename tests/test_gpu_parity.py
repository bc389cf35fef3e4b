"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Index sets must be bit-identical to the oracle's.  Products must match within
relative Frobenius error 5e-3 for bf16 inputs and 1e-5 for fp32 inputs.
Small cases span several tiles with ragged tails and are compared in full;
the full-size workloads are compared on every index and on sampled rows or
heads of the product (the selection always uses all rows).
"""

import numpy as np
import pytest
import torch

import synth
from input_adaptive_reduced_colnorm_amd import rmm
from oracle import rmm_oracle as O

pytestmark = pytest.mark.gpu

TOL_BF16 = 5e-3
TOL_FP32 = 1e-5


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    rmm.lib()
    return torch.device("cuda:0")


def f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of stored bf16 / fp32 values (numpy has no bf16)."""
    return t.detach().to("cpu").float().numpy()


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def run_matmul(A, B, rho, dev, out_dtype=torch.float32):
    idx, Y = rmm.matmul(A.to(dev), B.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), Y


def check_matmul(A, B, rho, dev, tol, out_dtype=torch.float32, rows=None):
    idx, Y = run_matmul(A, B, rho, dev, out_dtype)
    idx_o, Y_o = O.matmul(f32(A), f32(B), rho, rows=rows)
    assert idx.dtype == np.int32
    np.testing.assert_array_equal(idx, idx_o)
    Yg = f32(Y) if rows is None else f32(Y[torch.as_tensor(rows, device=Y.device)])
    err = rel_fro(Yg, Y_o)
    assert err <= tol, f"rel Frobenius error {err:.3e} > {tol}"
    return err


def check_matmul_w8(w, rho, dev, tol, out_dtype=torch.float32, rows=None):
    A, Bq, sc = w.tensors["A"], w.tensors["Bq"], w.tensors["scale"]
    print(f"matmul_w8 {tuple(A.shape)} x {tuple(Bq.shape)} rho={rho}", flush=True)
    idx, Y = rmm.matmul_w8(A.to(dev), Bq.to(dev), sc.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    idx_o, Y_o = O.matmul_w8(f32(A), Bq.numpy(), sc.numpy(), rho, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    Yg = f32(Y) if rows is None else f32(Y[torch.as_tensor(rows, device=Y.device)])
    err = rel_fro(Yg, Y_o)
    assert err <= tol, f"rel Frobenius error {err:.3e} > {tol}"


# ------------------------------- linear ------------------------------------

def test_tiny_projection_fp32(dev):
    w = synth.tiny_projection()
    check_matmul(w.tensors["A"], w.tensors["B"], 0.5, dev, TOL_FP32)
    check_matmul(w.tensors["A"], w.tensors["B"], 1.0, dev, TOL_FP32)


@pytest.mark.parametrize("rho", [0.9, 0.7, 0.5, 1.0])
def test_linear_bf16_ragged(dev, rho):
    # 300 x 1000 x 264: several 256-tiles in M, a ragged K tail, N tail
    w = synth.mlp_down(n=300, d=1000, m=264, rhos=(0.9, 0.7, 0.5))
    check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("rho", [0.7, 1.0])
def test_linear_bf16_output(dev, rho):
    w = synth.mlp_down(n=300, d=1000, m=264, rhos=(0.7,))
    check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16, out_dtype=torch.bfloat16)


def test_linear_odd_shapes(dev):
    # odd m rules out the 16-byte loaders: vector-ALU path on bf16 inputs
    w = synth.mlp_down(n=37, d=101, m=53, rhos=(0.6,))
    check_matmul(w.tensors["A"], w.tensors["B"], 0.6, dev, TOL_BF16)
    w = synth.mlp_down(n=33, d=77, m=40, rhos=(0.6,))
    check_matmul(w.tensors["A"], w.tensors["B"], 0.6, dev, TOL_BF16)
    check_matmul(w.tensors["A"], w.tensors["B"], 1.0, dev, TOL_BF16)


@pytest.mark.parametrize("rho", [0.7, 1.0])
def test_linear_leading_dims(dev, rho):
    w = synth.mlp_down(n=96, d=320, m=136, rhos=(0.7,))
    A, B = w.tensors["A"], w.tensors["B"]
    Aw = torch.zeros((96, 344), dtype=A.dtype)
    Aw[:, :320] = A
    Bw = torch.zeros((320, 160), dtype=B.dtype)
    Bw[:, :136] = B
    Ad, Bd = Aw.to(dev)[:, :320], Bw.to(dev)[:, :136]
    idx, Y = rmm.matmul(Ad, Bd, rho)
    torch.cuda.synchronize()
    idx_o, Y_o = O.matmul(f32(A), f32(B), rho)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    assert rel_fro(f32(Y), Y_o) <= TOL_BF16


def test_linear_unaligned_lda_dense(dev):
    # lda not a multiple of 8: rho = 1 goes through the gather-pack panel
    w = synth.mlp_down(n=64, d=200, m=72, rhos=(0.5,))
    A, B = w.tensors["A"], w.tensors["B"]
    Aw = torch.zeros((64, 203), dtype=A.dtype)
    Aw[:, :200] = A
    idx, Y = rmm.matmul(Aw.to(dev)[:, :200], B.to(dev), 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), np.arange(200))
    assert rel_fro(f32(Y), O.dense(f32(A), f32(B))) <= TOL_BF16


def test_edge_cases(dev):
    w = synth.mlp_down(n=40, d=100, m=48, rhos=(0.5,))
    A, B = w.tensors["A"], w.tensors["B"]
    check_matmul(A, B, 1e-6, dev, TOL_BF16)      # k = 1
    check_matmul(A, B, 0.999, dev, TOL_BF16)     # k = d with rho < 1
    check_matmul(A, B, 0.07, dev, TOL_BF16)      # k = 7 exactly (decimal reading)
    A1 = torch.randn(50, 1).to(torch.bfloat16)   # d = 1
    B1 = torch.randn(1, 16).to(torch.bfloat16)
    check_matmul(A1, B1, 0.5, dev, TOL_BF16)


def test_exact_ties_lowest_index(dev):
    # integer-valued columns with planted equal energies: lowest index wins
    r = np.random.default_rng(21)
    base = r.integers(-3, 4, size=(64, 16)).astype(np.float32)
    A = np.concatenate([base, base[:, ::-1], -base, np.zeros((64, 16), np.float32)], axis=1)
    B = r.standard_normal((64, 32)).astype(np.float32)
    for dt in (torch.float32, torch.bfloat16):
        At, Bt = torch.from_numpy(A).to(dt), torch.from_numpy(B).to(dt)
        for rho in (0.25, 0.3, 0.5, 0.8, 0.9):
            idx, _ = run_matmul(At, Bt, rho, dev)
            idx_o, _ = O.matmul(A, B, rho)
            np.testing.assert_array_equal(idx, idx_o)


@pytest.mark.parametrize("d", [64, 128, 192, 256, 320])
def test_linear_k_tile_counts(dev, d):
    # 1 to 5 K tiles of 64 through the linear GEMM's prefetch ring (direct A
    # rows two tiles ahead, per-iteration load counts), on the 256 x 256 tile
    # variant (4096 x 3072 output) and on the 128 x 128 one (300 x 264)
    for n, m in ((4096, 3072), (300, 264)):
        w = synth.mlp_down(n=n, d=d, m=m, rhos=(0.5,))
        A, B = w.tensors["A"], w.tensors["B"]
        for rho in (1.0, 0.5):
            check_matmul(A, B, rho, dev, TOL_BF16, rows=np.arange(0, n, 7) if n > 1000 else None)


@pytest.mark.parametrize("n,d", [(32, 3000), (32, 9000), (8, 4096)])
def test_radix_zero_and_tied_energies(dev, n, d):
    # integer entries give exact energies on both sides, with many ties; 40%
    # of the columns are zero, so large rho keeps every nonzero column plus
    # the lowest-indexed zero columns, and small rho never reaches the zeros.
    # d > 256 runs the radix selection (n = 8: the decode-shaped selection)
    r = np.random.default_rng(n * 7 + d)
    A = r.integers(-8, 9, size=(n, d)).astype(np.float32)
    A[:, r.random(d) < 0.4] = 0.0
    B = r.standard_normal((d, 16)).astype(np.float32)
    for rho in (0.1, 0.3, 0.5, 0.62, 0.7, 0.9):
        idx_o, _ = O.matmul(A, B, rho)
        At = torch.from_numpy(A).to(torch.bfloat16)
        idx = rmm.select(At.to(dev), rho)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        idx_m, _ = run_matmul(At, torch.from_numpy(B).to(torch.bfloat16), rho, dev)
        np.testing.assert_array_equal(idx_m, idx_o)


@pytest.mark.parametrize("n", [1, 5, 8, 16])
def test_decode_rows(dev, n):
    w = synth.decode_qkv(n=n, d=1024, m=776, rho=0.8)
    check_matmul(w.tensors["A"], w.tensors["B"], 0.8, dev, TOL_BF16)
    check_matmul(w.tensors["A"], w.tensors["B"], 1.0, dev, TOL_BF16)


def test_select_scores(dev):
    w = synth.mlp_down(n=200, d=700, m=8, rhos=(0.4,))
    A = w.tensors["A"]
    idx, s = rmm.select(A.to(dev), 0.4, scores=True)
    torch.cuda.synchronize()
    idx_o, q = O.select(f32(A), 0.4)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(s.cpu().numpy(), np.sqrt(q), rtol=1e-5)


@pytest.mark.parametrize("n,d", [(64, 200), (512, 3000), (40, 16000)])
def test_select_retained_energy(dev, n, d):
    # the three TopK paths: rank count (d <= 256), radix in LDS, radix in scratch
    w = synth.mlp_down(n=n, d=d, m=8, rhos=(0.7, 0.3))
    A = w.tensors["A"]
    for rho in (0.7, 0.3, 1.0):
        idx, ret = rmm.select_retained(A.to(dev), rho)
        torch.cuda.synchronize()
        idx_o, _ = O.select(f32(A), rho)
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        want = O.retained_energy(f32(A), rho)
        got = float(ret.cpu()[0])
        if rho == 1.0:
            assert got == 1.0
        assert abs(got - want) <= 1e-6 * want, (rho, got, want)


def test_determinism(dev):
    w = synth.mlp_down(n=512, d=2048, m=512, rhos=(0.7,))
    A, B = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
    i1, y1 = rmm.matmul(A, B, 0.7)
    i2, y2 = rmm.matmul(A, B, 0.7)
    w2 = synth.decode_qkv(n=8, d=2048, m=512, rho=0.8)
    A2, B2 = w2.tensors["A"].to(dev), w2.tensors["B"].to(dev)
    i3, y3 = rmm.matmul(A2, B2, 0.8)
    i4, y4 = rmm.matmul(A2, B2, 0.8)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(i3, i4) and torch.equal(y3.view(torch.int32), y4.view(torch.int32))


# ------------------------- given index list ---------------------------------

def _given_idx(d, k, seed):
    r = np.random.default_rng(seed)
    idx = r.choice(d, size=k, replace=True)                       # unsorted, with repeats
    idx[: max(1, k // 50)] = -5                                    # entries outside [0, d) are ignored
    idx[-1] = d + 7
    return idx.astype(np.int32)


@pytest.mark.parametrize("n", [300, 8])
def test_matmul_idx_selected_list_equals_reduced_product(dev, n):
    # the selected list handed back reproduces rmm_matmul bit for bit
    w = synth.mlp_down(n=n, d=1000, m=264, rhos=(0.7,))
    A, B = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
    idx, Y = rmm.matmul(A, B, 0.7)
    Y2 = rmm.matmul_idx(A, B, idx)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))


@pytest.mark.parametrize("n,dtype", [(300, torch.bfloat16), (8, torch.bfloat16), (40, torch.float32)])
def test_matmul_idx_arbitrary_list(dev, n, dtype):
    w = synth.mlp_down(n=n, d=700, m=136, rhos=(0.5,))
    A, B = w.tensors["A"].to(dtype), w.tensors["B"].to(dtype)
    idx = _given_idx(700, 450, seed=n)
    Y = rmm.matmul_idx(A.to(dev), B.to(dev), torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    ref = O.matmul_given(f32(A), f32(B), idx)
    err = rel_fro(f32(Y), ref)
    assert err <= (TOL_FP32 if dtype == torch.float32 else TOL_BF16), f"rel Frobenius error {err:.3e}"


def test_select_once_reuse_for_qkv(dev):
    # one selection on X serves three projections; each equals the matching
    # columns of the reduced product with the concatenated weights
    w = synth.mlp_down(n=256, d=1024, m=768, rhos=(0.6,))
    X, W = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
    idx = rmm.select(X, 0.6)
    _, Y = rmm.matmul(X, W, 0.6)
    for lo, hi in ((0, 512), (512, 640), (640, 768)):
        Yp = rmm.matmul_idx(X, W[:, lo:hi].contiguous(), idx)
        torch.cuda.synchronize()
        assert rel_fro(f32(Yp), f32(Y[:, lo:hi])) <= 1e-6


# --------------------------- int8 weights ----------------------------------

@pytest.mark.parametrize("rho", [0.8, 0.5, 1.0])
def test_matmul_w8_decode(dev, rho):
    # GEMV over the kept int8 rows: 3 and 16 activation rows, ragged strips
    w = synth.w8_projection(n=3, d=1000, m=264, rho=rho)
    check_matmul_w8(w, rho, dev, TOL_BF16)
    w = synth.w8_projection(n=16, d=2048, m=392, rho=rho)
    check_matmul_w8(w, rho, dev, TOL_BF16, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("rho", [0.7, 1.0])
def test_matmul_w8_prefill(dev, rho):
    # gathered int8 rows in the matrix-core GEMM: ragged M, K and N
    w = synth.w8_projection(n=300, d=700, m=520, rho=rho, name="w8_ragged")
    check_matmul_w8(w, rho, dev, TOL_BF16)
    # dense path with A read in place (d a multiple of 64), 256 x 256 tiles
    w = synth.w8_projection(n=1024, d=1024, m=768, rho=rho, name="w8_tiles")
    check_matmul_w8(w, rho, dev, TOL_BF16)


def test_full_mlp_down_w8(dev):
    # Llama-3.1-8B MLP down projection with int8 weights (256 x 256 tiles)
    w = synth.w8_projection(n=4096, d=14336, m=4096, rho=0.7, workload=1, name="mlp_down_8b_w8")
    rows = np.sort(np.random.default_rng(0).choice(4096, size=64, replace=False))
    check_matmul_w8(w, 0.7, dev, TOL_BF16, rows=rows)


def test_full_decode_qkv_w8(dev):
    w = synth.w8_projection()
    for rho in (0.8, 1.0):
        check_matmul_w8(w, rho, dev, TOL_BF16)


# -------------------------------- QK^T --------------------------------------

def check_qk(Q, K, rho, dev, tol, out_dtype=torch.float32):
    idx, S = rmm.qk(Q.to(dev), K.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    idx_o, S_o = O.qk(f32(Q), f32(K), rho)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    err = rel_fro(f32(S), S_o)
    assert err <= tol, f"rel Frobenius error {err:.3e}"


def check_qk_causal(Q, K, rho, dev, tol, out_dtype=torch.float32):
    idx, S = rmm.qk(Q.to(dev), K.to(dev), rho, out_dtype=out_dtype, causal=True)
    torch.cuda.synchronize()
    idx_o, S_o = O.qk(f32(Q), f32(K), rho, causal=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    Sg = f32(S)
    seen = np.isfinite(S_o)
    # -inf exactly where a key lies after the query position, finite elsewhere
    np.testing.assert_array_equal(np.isneginf(Sg), ~seen)
    assert np.all(np.isfinite(Sg[seen]))
    err = rel_fro(Sg[seen], S_o[seen])
    assert err <= tol, f"rel Frobenius error {err:.3e}"
    return S


@pytest.mark.parametrize("rho", [0.5, 1.0])
def test_qk_causal(dev, rho):
    # square (tq = tk) over several 128 x 128 tiles, whole tiles above the
    # diagonal skipped; then a chunk of 200 queries at the end of 520 keys
    w = synth.gqa_qk(hq=4, hkv=2, t=300, dh=128)
    check_qk_causal(w.tensors["Q"], w.tensors["K"], rho, dev, TOL_BF16)
    check_qk_causal(w.tensors["Q"], w.tensors["K"], rho, dev, TOL_BF16, out_dtype=torch.bfloat16)
    w = synth.gqa_qk(hq=4, hkv=1, t=520, dh=64)
    check_qk_causal(w.tensors["Q"][:, -200:, :].contiguous(), w.tensors["K"], rho, dev, TOL_BF16)


def test_qk_causal_large_tiles_fp32_and_decode(dev):
    # 256 x 256 tiles (16 heads x 1024 x 1024)
    w = synth.gqa_qk(hq=16, hkv=4, t=1024, dh=128)
    check_qk_causal(w.tensors["Q"], w.tensors["K"], 0.5, dev, TOL_BF16)
    # fp32 inputs (vector-ALU product) with a ragged head dim
    w = synth.gqa_qk(hq=4, hkv=2, t=70, dh=40)
    check_qk_causal(w.tensors["Q"].float(), w.tensors["K"].float(), 0.5, dev, TOL_FP32)
    # two new tokens against a cache (streaming pass over K)
    w = synth.decode_attn_qk(hq=8, hkv=2, tq=2, tk=1000, dh=128)
    check_qk_causal(w.tensors["Q"], w.tensors["K"], 0.5, dev, TOL_BF16)


def test_causal_prefill_attention_chain(dev):
    # causal scores -> softmax (1/sqrt(dh)) with key energies -> PV on them
    w = synth.gqa_qk(hq=4, hkv=2, t=384, dh=128)
    Q, K = w.tensors["Q"], w.tensors["K"]
    V = synth.attn_pv(h=4, hkv=2, tq=8, tk=384, dv=128).tensors["V"]
    # each stage against the oracle on the stage's own GPU input
    S = check_qk_causal(Q, K, 0.5, dev, TOL_BF16)
    P, E = check_softmax_energy(S.cpu(), dev, scale=128 ** -0.5)
    Pg = f32(P)
    assert np.all(Pg[np.isneginf(f32(S))] == 0.0)   # no weight after the query position
    idx, Og = rmm.pv_energy(P, V.to(dev), E, 0.5)
    torch.cuda.synchronize()
    idx_o, O_o = O.pv_given_energy(Pg, f32(V), f32(E), 0.5)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    assert rel_fro(f32(Og), O_o) <= TOL_BF16


@pytest.mark.parametrize("rho", [0.5, 1.0])
def test_qk_small(dev, rho):
    w = synth.gqa_qk(hq=4, hkv=2, t=300, dh=128)
    check_qk(w.tensors["Q"], w.tensors["K"], rho, dev, TOL_BF16)


def test_qk_fp32_and_odd(dev):
    w = synth.gqa_qk(hq=4, hkv=1, t=70, dh=64)
    Q, K = w.tensors["Q"].float(), w.tensors["K"].float()
    check_qk(Q, K, 0.5, dev, TOL_FP32)
    w = synth.gqa_qk(hq=6, hkv=3, t=45, dh=40)  # dh not a multiple of 64
    check_qk(w.tensors["Q"], w.tensors["K"], 0.5, dev, TOL_BF16)
    check_qk(w.tensors["Q"], w.tensors["K"], 0.5, dev, TOL_BF16, out_dtype=torch.bfloat16)


def test_qk_wide_head(dev):
    # dh = 256 at rho 0.7: k = 180, padded to 192 (24 packed pieces per row)
    w = synth.gqa_qk(hq=4, hkv=2, t=130, dh=256)
    check_qk(w.tensors["Q"], w.tensors["K"], 0.7, dev, TOL_BF16)


@pytest.mark.parametrize("d", [255, 256, 257])
def test_selection_size_boundary(dev, d):
    # d <= 256 selects with the rank kernel, larger d with the radix kernel
    w = synth.mlp_down(n=96, d=d, m=72, rhos=(0.5, 0.3))
    for rho in (0.5, 0.3):
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


# --------------------------------- PV ---------------------------------------

def check_pv(P, V, rho, dev, tol, heads=None):
    idx, Og = rmm.pv(P.to(dev), V.to(dev), rho)
    torch.cuda.synchronize()
    hs = list(range(P.shape[0])) if heads is None else list(heads)
    idx_o, O_o = O.pv(f32(P), f32(V), rho, heads=hs)
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi[hs], idx_o)
    err = rel_fro(f32(Og[torch.as_tensor(hs, device=Og.device)]), O_o)
    assert err <= tol, f"rel Frobenius error {err:.3e}"
    return gi


@pytest.mark.parametrize("rho", [0.5, 1.0])
def test_pv_small(dev, rho):
    w = synth.attn_pv(h=4, hkv=2, tq=100, tk=1000, dv=128)
    check_pv(w.tensors["P"], w.tensors["V"], rho, dev, TOL_BF16)
    check_pv(w.tensors["P"].to(torch.bfloat16), w.tensors["V"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("rho", [0.5, 0.2, 0.1])
def test_pv_masked_and_packed(dev, rho):
    # tk = 1024: rho 0.5 and 0.2 keep at least one key in eight (P read in
    # place, dropped V rows masked); rho 0.1 keeps fewer (kept P packed)
    w = synth.attn_pv(h=4, hkv=2, tq=96, tk=1024, dv=64, rho=rho)
    check_pv(w.tensors["P"], w.tensors["V"], rho, dev, TOL_BF16)
    check_pv(w.tensors["P"].to(torch.bfloat16), w.tensors["V"], rho, dev, TOL_BF16)


# ------------------- producer-side PV scoring (softmax) ----------------------

def check_softmax_energy(L, dev, heads=None, scale=1.0):
    P, E = rmm.softmax_energy(L.to(dev), scale)
    torch.cuda.synchronize()
    hs = list(range(L.shape[0])) if heads is None else list(heads)
    Pg = f32(P[torch.as_tensor(hs, device=P.device)])
    Po = O.softmax_rows(f32(L[hs]), scale)
    err = rel_fro(Pg, Po)
    assert err <= 1e-6, f"softmax rel Frobenius error {err:.3e}"
    assert np.max(np.abs(Pg - Po)) <= 1e-6 * np.max(Po)
    # the energies are those of the P the kernel wrote
    Eo = np.stack([O.col_energy(Pg[i]) for i in range(len(hs))])
    e_err = rel_fro(f32(E[torch.as_tensor(hs, device=E.device)]), Eo)
    assert e_err <= 1e-5, f"energy rel error {e_err:.3e}"
    return P, E


@pytest.mark.parametrize("rho", [0.5, 0.2])
def test_softmax_energy_then_pv(dev, rho):
    w = synth.attn_pv(h=4, hkv=2, tq=96, tk=1024, dv=64, rho=rho, with_logits=True)
    P, E = check_softmax_energy(w.tensors["L"], dev)
    V = w.tensors["V"].to(dev)
    idx, Og = rmm.pv_energy(P, V, E, rho)
    torch.cuda.synchronize()
    Pc = f32(P)
    idx_o, O_o = O.pv_given_energy(Pc, f32(w.tensors["V"]), f32(E), rho)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    assert rel_fro(f32(Og), O_o) <= TOL_BF16
    # the same keys and product as PV scoring P itself
    idx2, O2 = rmm.pv(P, V, rho)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(Og.view(torch.int32), O2.view(torch.int32))


def test_softmax_energy_odd_sizes(dev):
    r = np.random.default_rng(3)
    for h, tq, tk in ((3, 5, 77), (2, 33, 300), (1, 7, 2500)):
        L = torch.from_numpy(r.normal(0.0, 2.0, size=(h, tq, tk)).astype(np.float32))
        check_softmax_energy(L, dev)
        check_softmax_energy(L, dev, scale=0.125)


def test_pv_fp32(dev):
    w = synth.attn_pv(h=2, hkv=1, tq=40, tk=300, dv=24)
    check_pv(w.tensors["P"], w.tensors["V"].float(), 0.5, dev, TOL_FP32)


# ------------------------- decode attention ----------------------------------

@pytest.mark.parametrize("tq,dh,rho", [(1, 128, 0.5), (1, 128, 1.0), (2, 64, 0.5), (1, 256, 0.7), (1, 40, 0.5)])
def test_qk_decode(dev, tq, dh, rho):
    # streaming pass over the key cache (tq <= 16 and group * tq <= 8), and
    # the pack + GEMM path for a head dim the streaming pass does not take
    w = synth.decode_attn_qk(hq=8, hkv=2, tq=tq, tk=1000, dh=dh)
    check_qk(w.tensors["Q"], w.tensors["K"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("tq,dh,rho", [(1, 128, 0.5), (2, 64, 0.3), (1, 256, 0.7), (1, 128, 0.9)])
def test_qk_decode_tied_energies(dev, tq, dh, rho):
    # queries drawn from {0, +-1, +-2}: most feature energies tie and many are
    # zero, so the kept set is decided by the lowest-index rule; the streaming
    # kernel's in-kernel ranking must give the oracle's lists exactly
    w = synth.decode_attn_qk(hq=8, hkv=2, tq=tq, tk=600, dh=dh)
    g = torch.Generator().manual_seed(11)
    vals = torch.tensor([0.0, 0.0, 1.0, -1.0, 2.0, -2.0])
    Q = vals[torch.randint(0, len(vals), w.tensors["Q"].shape, generator=g)].to(torch.bfloat16)
    check_qk(Q, w.tensors["K"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("tq,rho", [(1, 0.5), (1, 1.0), (4, 0.3)])
def test_pv_decode(dev, tq, rho):
    # a GEMV per head over the kept rows of V
    w = synth.attn_pv(h=8, hkv=2, tq=tq, tk=1000, dv=128, rho=rho, with_logits=True)
    check_pv(w.tensors["P"], w.tensors["V"], rho, dev, TOL_BF16)
    check_pv(w.tensors["P"].to(torch.bfloat16), w.tensors["V"], rho, dev, TOL_BF16)
    # with the energies from the softmax pass
    P, E = check_softmax_energy(w.tensors["L"], dev)
    idx, Og = rmm.pv_energy(P, w.tensors["V"].to(dev), E, rho)
    torch.cuda.synchronize()
    idx_o, O_o = O.pv_given_energy(f32(P), f32(w.tensors["V"]), f32(E), rho)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    assert rel_fro(f32(Og), O_o) <= TOL_BF16


def test_full_decode_attention(dev):
    # Llama-3.1-8B decode step: 32 query heads, 8 kv heads, 8192 cached tokens
    wq = synth.decode_attn_qk(hq=32, hkv=8, tq=1, tk=8192, dh=128)
    check_qk(wq.tensors["Q"], wq.tensors["K"], 0.5, dev, TOL_BF16)
    wp = synth.attn_pv(h=32, hkv=8, tq=1, tk=8192, dv=128, rho=0.5)
    check_pv(wp.tensors["P"], wp.tensors["V"], 0.5, dev, TOL_BF16)


# ----------------------------- full sizes -----------------------------------

def test_full_mlp_down(dev):
    w = synth.mlp_down()
    A, B = w.tensors["A"], w.tensors["B"]
    rows = np.random.default_rng(0).choice(A.shape[0], size=96, replace=False)
    rows.sort()
    for rho in (0.9, 0.7, 0.5, 1.0):
        print(f"mlp_down 4096x14336x4096 rho={rho}", flush=True)
        check_matmul(A, B, rho, dev, TOL_BF16, rows=rows)


def test_full_decode_qkv(dev):
    w = synth.decode_qkv()
    for rho in (0.8, 1.0):
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


def test_full_mlp_up(dev):
    w = synth.mlp_up()
    rows = np.random.default_rng(1).choice(2048, size=48, replace=False)
    rows.sort()
    for rho in (0.8, 1.0):
        print(f"mlp_up 2048x8192x28672 rho={rho}", flush=True)
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16, rows=rows)


def test_full_gqa_qk(dev):
    w = synth.gqa_qk()
    Q, K = w.tensors["Q"], w.tensors["K"]
    for rho in (0.5, 1.0):
        print(f"gqa_qk 32x4096x128 rho={rho}", flush=True)
        idx, S = rmm.qk(Q.to(dev), K.to(dev), rho)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        for h in range(Q.shape[0]):   # every head's index set
            ih, _ = O.select(f32(Q[h]), rho)
            np.testing.assert_array_equal(gi[h], ih)
        hs = [0, 5, 17, 31]
        _, S_o = O.qk(f32(Q), f32(K), rho, heads=hs)
        err = rel_fro(f32(S[torch.as_tensor(hs, device=S.device)]), S_o)
        assert err <= TOL_BF16, err
        del S


def test_full_attn_pv_with_producer(dev):
    w = synth.attn_pv(with_logits=True)
    heads = [0, 9, 37, 63]
    P, E = check_softmax_energy(w.tensors["L"], dev, heads=heads)
    idx, Og = rmm.pv_energy(P, w.tensors["V"].to(dev), E, 0.5)
    torch.cuda.synchronize()
    hi = torch.as_tensor(heads)
    Pc = f32(P[hi.to(P.device)])
    Eo = np.stack([O.col_energy(Pc[i]) for i in range(len(heads))])
    order = [np.sort(np.argsort(-Eo[i], kind="stable")[:O.k_rule(0.5, Pc.shape[2])]) for i in range(len(heads))]
    np.testing.assert_array_equal(idx.cpu().numpy()[heads], np.stack(order))
    Vc = f32(w.tensors["V"])
    for i, h in enumerate(heads):
        g = O.kv_head(h, 64, 8)
        ref = Pc[i][:, order[i]].astype(np.float64) @ Vc[g][order[i], :].astype(np.float64)
        assert rel_fro(f32(Og[h]), ref) <= TOL_BF16


def test_full_attn_pv(dev):
    w = synth.attn_pv()
    P, V = w.tensors["P"], w.tensors["V"]
    for rho in (0.5, 1.0):
        print(f"attn_pv 64x512x8192 rho={rho}", flush=True)
        idx, Og = rmm.pv(P.to(dev), V.to(dev), rho)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        Pn = f32(P)
        for h in range(P.shape[0]):
            ih, _ = O.select(Pn[h], rho)
            np.testing.assert_array_equal(gi[h], ih)
        hs = [0, 9, 40, 63]
        _, O_o = O.pv(Pn, f32(V), rho, heads=hs)
        err = rel_fro(f32(Og[torch.as_tensor(hs, device=Og.device)]), O_o)
        assert err <= TOL_BF16, err
