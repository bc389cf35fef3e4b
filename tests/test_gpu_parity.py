"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Index sets must be bit-identical to the oracle's.  Products must match within
relative Frobenius error 5e-3 for bf16 inputs and 1e-5 for fp32 inputs, and
every compared element must also lie within the same tolerance times its
magnitude envelope, |Y - Y_o|_ij <= tol * (|A_I| |B_I|)_ij: the sum of the
absolute values of the terms the element adds up, which bounds both the
float32 accumulation error and a bf16 rounding of the output, so a single
wrong element, tile edge or epilogue lane fails even where the norm would
hide it.  Small cases span several tiles with ragged tails and are compared
in full; the full-size workloads are compared on every index and on rows
chosen so that every 256-row tile and every row position inside a 32-row
MFMA block is covered, over all columns (the selection always uses all
rows).
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
# two roundings to bf16 (nearest even, each at most 2**-8 of the element's
# envelope): fp32 P staged as bf16 for the matrix cores, then a bf16 output
TOL_BF16_TWICE = 8e-3


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


def envelope(A, B, idx, rows=None) -> np.ndarray:
    """(|A[:, I]| |B[I, :]|)_ij in float64: the magnitude scale of element
    (i, j) of the reduced product (entries of idx outside [0, d) skipped, a
    repeated entry counted per occurrence).  A tolerance scale, not an
    expected value."""
    A64 = np.abs(np.asarray(A, dtype=np.float64))
    B64 = np.abs(np.asarray(B, dtype=np.float64))
    I = np.asarray(idx, dtype=np.int64).ravel()
    I = I[(I >= 0) & (I < A64.shape[1])]
    Ar = A64 if rows is None else A64[np.asarray(rows)]
    return Ar[:, I] @ B64[I, :]


def assert_close(got, ref, env, tol, what="product"):
    """Relative Frobenius error <= tol, and |got - ref| <= tol * env for
    every element (env: the magnitude envelope of each element)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    env = np.asarray(env, dtype=np.float64)
    assert got.shape == ref.shape == env.shape, (got.shape, ref.shape, env.shape)
    err = rel_fro(got, ref)
    assert err <= tol, f"{what}: rel Frobenius error {err:.3e} > {tol}"
    diff = np.abs(got - ref)
    bad = ~(diff <= tol * env)          # also catches NaN
    if bad.any():
        at = np.unravel_index(int(np.argmax(np.where(bad, diff - tol * env, -np.inf))), bad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside tol*envelope; worst at {at}: "
                             f"got {got[at]!r} want {ref[at]!r} envelope {env[at]!r}")
    return err


def tile_rows(n: int, tile: int = 256) -> np.ndarray:
    """Rows that cover every row tile and every row position within a
    32-row block (the accumulator lanes of the epilogue), plus each tile's
    first and last row."""
    offs = sorted(set(range(32)) | {45, 64, 100, 127, 128, 170, 203, 230, 254, tile - 1})
    rows = {t + o for t in range(0, n, tile) for o in offs if o < tile and t + o < n}
    rows.add(n - 1)
    return np.array(sorted(rows), dtype=np.int64)


def run_matmul(A, B, rho, dev, out_dtype=torch.float32):
    idx, Y = rmm.matmul(A.to(dev), B.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), Y


def check_matmul(A, B, rho, dev, tol, out_dtype=torch.float32, rows=None):
    idx, Y = run_matmul(A, B, rho, dev, out_dtype)
    Af, Bf = f32(A), f32(B)
    idx_o, Y_o = O.matmul(Af, Bf, rho, rows=rows)
    assert idx.dtype == np.int32
    np.testing.assert_array_equal(idx, idx_o)
    Yg = f32(Y) if rows is None else f32(Y[torch.as_tensor(rows, device=Y.device)])
    return assert_close(Yg, Y_o, envelope(Af, Bf, idx_o, rows), tol)


def check_matmul_w8(w, rho, dev, tol, out_dtype=torch.float32, rows=None):
    A, Bq, sc = w.tensors["A"], w.tensors["Bq"], w.tensors["scale"]
    print(f"matmul_w8 {tuple(A.shape)} x {tuple(Bq.shape)} rho={rho}", flush=True)
    idx, Y = rmm.matmul_w8(A.to(dev), Bq.to(dev), sc.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    Af = f32(A)
    idx_o, Y_o = O.matmul_w8(Af, Bq.numpy(), sc.numpy(), rho, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    Yg = f32(Y) if rows is None else f32(Y[torch.as_tensor(rows, device=Y.device)])
    Bs = Bq.numpy().astype(np.float64) * sc.numpy().astype(np.float64)[None, :]
    assert_close(Yg, Y_o, envelope(Af, Bs, idx_o, rows), tol)


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
    assert_close(f32(Y), Y_o, envelope(f32(A), f32(B), idx_o), TOL_BF16)


def test_linear_unaligned_lda_dense(dev):
    # lda not a multiple of 8: rho = 1 goes through the gather-pack panel
    w = synth.mlp_down(n=64, d=200, m=72, rhos=(0.5,))
    A, B = w.tensors["A"], w.tensors["B"]
    Aw = torch.zeros((64, 203), dtype=A.dtype)
    Aw[:, :200] = A
    idx, Y = rmm.matmul(Aw.to(dev)[:, :200], B.to(dev), 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), np.arange(200))
    assert_close(f32(Y), O.dense(f32(A), f32(B)), envelope(f32(A), f32(B), np.arange(200)), TOL_BF16)


def test_linear_column_offset_view_dense(dev):
    # A = X[:, 1:65] of a 72-wide X: 2-byte aligned only, so rho = 1 cannot
    # read A in place and packs it; the workspace query must cover that
    w = synth.mlp_down(n=96, d=64, m=40, rhos=(0.5,))
    A, B = w.tensors["A"], w.tensors["B"]
    X = torch.zeros((96, 72), dtype=A.dtype)
    X[:, 1:65] = A
    Xd = X.to(dev)
    for rho in (1.0, 0.5):
        idx, Y = rmm.matmul(Xd[:, 1:65], B.to(dev), rho)
        torch.cuda.synchronize()
        idx_o, Y_o = O.matmul(f32(A), f32(B), rho)
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        assert_close(f32(Y), Y_o, envelope(f32(A), f32(B), idx_o), TOL_BF16)


def test_edge_cases(dev):
    w = synth.mlp_down(n=40, d=100, m=48, rhos=(0.5,))
    A, B = w.tensors["A"], w.tensors["B"]
    check_matmul(A, B, 1e-6, dev, TOL_BF16)      # k = 1
    check_matmul(A, B, 0.999, dev, TOL_BF16)     # k = d with rho < 1
    check_matmul(A, B, 0.07, dev, TOL_BF16)      # k = 7 exactly (decimal reading)
    g = torch.Generator().manual_seed(5)
    A1 = torch.randn(50, 1, generator=g).to(torch.bfloat16)   # d = 1
    B1 = torch.randn(1, 16, generator=g).to(torch.bfloat16)
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


@pytest.mark.parametrize("n,d,rho", [(17, 8, 0.5), (257, 8200, 0.9), (300, 15360, 0.999), (64, 4096, 1e-6),
                                     (1000, 2048, 0.5), (4100, 15360, 0.7)])
def test_fused_selection_gather_shapes(dev, n, d, rho):
    # the one-launch selection + gather of the prefill products: one row
    # block per workgroup (a short last block when n is not a multiple of
    # it), rows of one 16-byte piece up to the 15360-column key capacity,
    # waves with one or two row loads (d = 8200), k = 1 and k = d - 15
    w = synth.mlp_down(n=n, d=d, m=72, rhos=(rho,))
    print(f"fused selection+gather n={n} d={d} rho={rho}", flush=True)
    rows = tile_rows(n) if n > 1000 else None
    check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16, rows=rows)


def test_fused_and_separate_selection_agree_bitwise(dev):
    # the one-launch ranking + gather and the separate TopK + pack launches
    # (taken when rows are not whole 16-byte pieces: a row stride of d + 3)
    # feed the same GEMM, so their kept lists and products agree bit for bit;
    # likewise for QK^T heads and for a given index list
    w = synth.mlp_down(n=600, d=2048, m=264, rhos=(0.7,))
    A, B = w.tensors["A"], w.tensors["B"]
    X = torch.zeros((600, 2051), dtype=A.dtype)
    X[:, :2048] = A
    Ad, Xd, Bd = A.to(dev), X.to(dev)[:, :2048], B.to(dev)
    for rho in (0.7, 0.3):
        i1, Y1 = rmm.matmul(Ad, Bd, rho)
        i2, Y2 = rmm.matmul(Xd, Bd, rho)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2)
        assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
        g1 = rmm.matmul_idx(Ad, Bd, i1)
        g2 = rmm.matmul_idx(Xd, Bd, i1)
        torch.cuda.synchronize()
        assert torch.equal(g1.view(torch.int32), Y1.view(torch.int32))
        assert torch.equal(g2.view(torch.int32), Y1.view(torch.int32))
    q = synth.gqa_qk(hq=8, hkv=2, t=260, dh=128)
    Q, K = q.tensors["Q"], q.tensors["K"]
    Qw = torch.zeros((8, 260, 131), dtype=Q.dtype)
    Kw = torch.zeros((2, 260, 131), dtype=K.dtype)
    Qw[:, :, :128] = Q
    Kw[:, :, :128] = K
    j1, S1 = rmm.qk(Q.to(dev), K.to(dev), 0.5)
    j2, S2 = rmm.qk(Qw.to(dev)[:, :, :128], Kw.to(dev)[:, :, :128], 0.5)
    torch.cuda.synchronize()
    assert torch.equal(j1, j2)
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))


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


@pytest.mark.parametrize("n,d", [(64, 300), (64, 4096), (8, 4096), (24, 20000)])
def test_equal_nonzero_energies(dev, n, d):
    # +-1 entries: every nonzero column has energy n exactly and a third of
    # the columns are zero, so the radix search finds no spread among the
    # nonzero keys (or k beyond them) and decides by index alone: rho below
    # the nonzero share keeps the lowest-indexed nonzero columns, above it
    # every nonzero column plus the lowest-indexed zero ones.  d = 300 and
    # 4096 run the LDS radix kernel, n = 8 the decode selection, d = 20000
    # the scratch-memory radix kernel.
    r = np.random.default_rng(d + n)
    A = np.where(r.random((n, d)) < 0.5, 1.0, -1.0).astype(np.float32)
    A[:, r.random(d) < 0.33] = 0.0
    B = r.standard_normal((d, 24)).astype(np.float32)
    At = torch.from_numpy(A).to(torch.bfloat16)
    for rho in (0.2, 0.5, 0.66, 0.9):
        idx_o, _ = O.select(A, rho)
        idx = rmm.select(At.to(dev), rho)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        check_matmul(At, torch.from_numpy(B).to(torch.bfloat16), rho, dev, TOL_BF16)


def test_pv_uniform_rows(dev):
    # uniform attention rows: every key position has the same energy, so the
    # lowest positions are kept; tk = 512 takes the radix selection
    P = torch.full((4, 16, 512), 1.0 / 512.0, dtype=torch.float32)
    V = synth.attn_pv(h=4, hkv=2, tq=16, tk=512, dv=64).tensors["V"]
    for rho in (0.5, 0.3):
        gi = check_pv(P, V, rho, dev, TOL_BF16)
        np.testing.assert_array_equal(gi, np.tile(np.arange(O.k_rule(rho, 512)), (4, 1)))


@pytest.mark.parametrize("n", [1, 5, 8, 16])
def test_decode_rows(dev, n):
    w = synth.decode_qkv(n=n, d=1024, m=776, rho=0.8)
    check_matmul(w.tensors["A"], w.tensors["B"], 0.8, dev, TOL_BF16)
    check_matmul(w.tensors["A"], w.tensors["B"], 1.0, dev, TOL_BF16)


@pytest.mark.parametrize("n,d", [(8, 1001), (3, 4104), (16, 8192), (8, 9000)])
def test_decode_row_widths(dev, n, d):
    # the GEMV ranks the columns itself with 16 keys per thread (d <= 4096;
    # d = 1001 takes the element loads), 32 keys (d <= 8192); wider rows run
    # the selection kernel first
    w = synth.decode_qkv(n=n, d=d, m=520, rho=0.7)
    for rho in (0.7, 1.0):
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("n,d,m,rho", [(4, 96, 520, 0.5), (8, 8192, 264, 0.3), (8, 4096, 6144, 0.95),
                                       (16, 8192, 1032, 0.1), (1, 5000, 776, 0.7), (16, 4100, 264, 0.6)])
def test_decode_source_slices(dev, n, d, m, rho):
    # the GEMV that ranks A itself owns ranges of B's source rows: slices
    # shorter than the 128 rows requested before the ranking (d = 96; d =
    # 8192 with 3 column strips gives 128-row slices), the rest of a slice
    # after them (d = 4096: 416-row slices), a ragged last slice and column
    # strip (m = 1032), most rows of the early part dropped or kept (rho 0.1,
    # 0.95), element loads of A (d = 5000, 4100: 20 and 17 columns per
    # thread), 16 activation rows with 32 keys per thread
    w = synth.decode_qkv(n=n, d=d, m=m, rho=rho)
    check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("n,d,m", [(8, 4096, 520), (300, 2048, 264), (16, 8192, 264)])
def test_dropped_rows_of_b_never_reach_the_product(dev, n, d, m):
    # the decode GEMV requests each slice's first rows before it knows which
    # are kept and zeroes the dropped ones on both operands; the prefill
    # GEMM gathers only kept rows: NaN in every dropped row of B must leave
    # Y and idx exactly as with zeros there
    w = synth.decode_qkv(n=n, d=d, m=m, rho=0.6)
    A, B = w.tensors["A"], w.tensors["B"]
    idx_o, _ = O.select(f32(A), 0.6)
    drop = np.setdiff1d(np.arange(d), idx_o)
    Bz, Bn = B.clone(), B.clone()
    Bz[drop] = 0
    Bn[drop] = float("nan")
    i1, y1 = rmm.matmul(A.to(dev), Bz.to(dev), 0.6)
    i2, y2 = rmm.matmul(A.to(dev), Bn.to(dev), 0.6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(i1.cpu().numpy(), idx_o)
    assert torch.equal(i1, i2)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_decode_ranked_unaligned_view(dev):
    # a column-offset view of A (rows not 16-byte aligned) takes the element
    # loads of the in-GEMV ranking and stages the slice's activations from them
    w = synth.decode_qkv(n=8, d=2048, m=520, rho=0.7)
    A, B = w.tensors["A"], w.tensors["B"]
    X = torch.zeros((8, 2051), dtype=A.dtype)
    X[:, 3:] = A
    idx, Y = rmm.matmul(X.to(dev)[:, 3:], B.to(dev), 0.7)
    torch.cuda.synchronize()
    idx_o, Y_o = O.matmul(f32(A), f32(B), 0.7)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    assert_close(Y.cpu().numpy(), Y_o, envelope(f32(A), f32(B), idx_o), TOL_BF16)


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
    # the selected list handed back reproduces rmm_matmul: bit for bit on
    # the prefill path (the same packed panel and GEMM); on the decode path
    # the GEMV that ranks A itself slices the source rows of B while the
    # given-list GEMV slices the list, so their fp32 sums of the same bf16
    # products are grouped differently and agree to fp32 rounding
    w = synth.mlp_down(n=n, d=1000, m=264, rhos=(0.7,))
    A, B = w.tensors["A"].to(dev), w.tensors["B"].to(dev)
    idx, Y = rmm.matmul(A, B, 0.7)
    Y2 = rmm.matmul_idx(A, B, idx)
    torch.cuda.synchronize()
    if n > 16:
        assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    else:
        env = envelope(f32(A), f32(B), idx.cpu().numpy())
        assert_close(Y2.cpu().numpy(), Y.cpu().numpy(), env, 1e-5, "given list vs ranked in the GEMV")


@pytest.mark.parametrize("n,dtype", [(300, torch.bfloat16), (8, torch.bfloat16), (40, torch.float32)])
def test_matmul_idx_arbitrary_list(dev, n, dtype):
    w = synth.mlp_down(n=n, d=700, m=136, rhos=(0.5,))
    A, B = w.tensors["A"].to(dtype), w.tensors["B"].to(dtype)
    idx = _given_idx(700, 450, seed=n)
    Y = rmm.matmul_idx(A.to(dev), B.to(dev), torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    ref = O.matmul_given(f32(A), f32(B), idx)
    assert_close(f32(Y), ref, envelope(f32(A), f32(B), idx), TOL_FP32 if dtype == torch.float32 else TOL_BF16)


@pytest.mark.parametrize("n,d,k", [(300, 1000, 450), (300, 1000, 1500), (257, 4096, 9000), (64, 2048, 16000)])
def test_matmul_idx_whole_row_gather(dev, n, d, k):
    # given lists on rows of whole 16-byte pieces (the one-launch gather
    # through LDS): unsorted, repeated and out-of-range entries; lists longer
    # than d, one with more entries than the 8192 a thread pair holds for
    # rows of 4096 columns, and one past the LDS list capacity (the
    # element-gather pack instead)
    w = synth.mlp_down(n=n, d=d, m=136, rhos=(0.5,))
    A, B = w.tensors["A"], w.tensors["B"]
    idx = _given_idx(d, k, seed=k)
    print(f"matmul_idx n={n} d={d} k={k}", flush=True)
    Y = rmm.matmul_idx(A.to(dev), B.to(dev), torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    ref = O.matmul_given(f32(A), f32(B), idx)
    assert_close(f32(Y), ref, envelope(f32(A), f32(B), idx), TOL_BF16)


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
    check_matmul_w8(w, 0.7, dev, TOL_BF16, rows=tile_rows(4096))


def test_full_decode_qkv_w8(dev):
    w = synth.w8_projection()
    for rho in (0.8, 1.0):
        check_matmul_w8(w, rho, dev, TOL_BF16)


# -------------------------------- QK^T --------------------------------------

def qk_envelope(Q, K, idx, heads=None) -> np.ndarray:
    """Per head, |Q[h][:, I_h]| |K[g(h)][:, I_h]|^T (the magnitude scale of
    each score)."""
    hq, hkv = Q.shape[0], K.shape[0]
    hs = range(hq) if heads is None else heads
    return np.stack([envelope(Q[h], np.asarray(K[h // (hq // hkv)]).T, idx[i]) for i, h in enumerate(hs)])


def check_qk(Q, K, rho, dev, tol, out_dtype=torch.float32):
    idx, S = rmm.qk(Q.to(dev), K.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    Qf, Kf = f32(Q), f32(K)
    idx_o, S_o = O.qk(Qf, Kf, rho)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    assert_close(f32(S), S_o, qk_envelope(Qf, Kf, idx_o), tol, "scores")


def check_qk_causal(Q, K, rho, dev, tol, out_dtype=torch.float32):
    idx, S = rmm.qk(Q.to(dev), K.to(dev), rho, out_dtype=out_dtype, causal=True)
    torch.cuda.synchronize()
    Qf, Kf = f32(Q), f32(K)
    idx_o, S_o = O.qk(Qf, Kf, rho, causal=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    Sg = f32(S)
    seen = np.isfinite(S_o)
    # -inf exactly where a key lies after the query position, finite elsewhere
    np.testing.assert_array_equal(np.isneginf(Sg), ~seen)
    assert np.all(np.isfinite(Sg[seen]))
    assert_close(Sg[seen], S_o[seen], qk_envelope(Qf, Kf, idx_o)[seen], tol, "causal scores")
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
    assert_close(f32(Og), O_o, pv_envelope(Pg, f32(V), idx_o), TOL_BF16, "PV")


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


def test_qk_strided_heads(dev):
    # Q and K as views of token-major [t][heads][dh] buffers (head stride dh,
    # row stride heads * dh), then of rows padded to 152 elements, both
    # through the one-launch feature selection and gather; rows padded to
    # 131 elements (not whole 16-byte pieces) take the separate TopK and
    # element-gather packs
    w = synth.gqa_qk(hq=8, hkv=2, t=200, dh=128)
    Q, K = w.tensors["Q"], w.tensors["K"]
    Qf, Kf = f32(Q), f32(K)
    idx_o, S_o = O.qk(Qf, Kf, 0.5)
    env = qk_envelope(Qf, Kf, idx_o)
    views = [(Q.permute(1, 0, 2).contiguous().to(dev).permute(1, 0, 2),
              K.permute(1, 0, 2).contiguous().to(dev).permute(1, 0, 2))]
    for width in (152, 131):
        Qw = torch.zeros((8, 200, width), dtype=Q.dtype)
        Kw = torch.zeros((2, 200, width), dtype=K.dtype)
        Qw[:, :, :128] = Q
        Kw[:, :, :128] = K
        views.append((Qw.to(dev)[:, :, :128], Kw.to(dev)[:, :, :128]))
    for Qd, Kd in views:
        print(f"qk strides Q {Qd.stride()} K {Kd.stride()}", flush=True)
        idx, S = rmm.qk(Qd, Kd, 0.5)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        assert_close(f32(S), S_o, env, TOL_BF16, "scores")


@pytest.mark.parametrize("d", [255, 256, 257])
def test_selection_size_boundary(dev, d):
    # d <= 256 selects with the rank kernel, larger d with the radix kernel
    w = synth.mlp_down(n=96, d=d, m=72, rhos=(0.5, 0.3))
    for rho in (0.5, 0.3):
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


# --------------------------------- PV ---------------------------------------

def pv_envelope(P, V, idx, heads=None) -> np.ndarray:
    """Per head, |P[h][:, I_h]| |V[g(h)][I_h, :]|."""
    h_, hkv = P.shape[0], V.shape[0]
    hs = range(h_) if heads is None else heads
    return np.stack([envelope(P[h], V[h // (h_ // hkv)], idx[i]) for i, h in enumerate(hs)])


def check_pv(P, V, rho, dev, tol, heads=None, out_dtype=torch.float32):
    idx, Og = rmm.pv(P.to(dev), V.to(dev), rho, out_dtype=out_dtype)
    torch.cuda.synchronize()
    hs = list(range(P.shape[0])) if heads is None else list(heads)
    Pf, Vf = f32(P), f32(V)
    idx_o, O_o = O.pv(Pf, Vf, rho, heads=hs)
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi[hs], idx_o)
    assert_close(f32(Og[torch.as_tensor(hs, device=Og.device)]), O_o, pv_envelope(Pf, Vf, idx_o, hs), tol, "PV")
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
    # where fp32 P is read in place (rho 0.5, 0.2) the contraction of its 4
    # tiles runs in 4 ranges: their ordered sum also rounds to a bf16 output,
    # a second rounding after that of P
    check_pv(w.tensors["P"], w.tensors["V"], rho, dev, TOL_BF16_TWICE, out_dtype=torch.bfloat16)


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
    assert_close(f32(Og), O_o, pv_envelope(Pc, f32(w.tensors["V"]), idx_o), TOL_BF16, "PV")
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
    assert_close(f32(Og), O_o, pv_envelope(f32(P), f32(w.tensors["V"]), idx_o), TOL_BF16, "PV")


def test_full_decode_attention(dev):
    # Llama-3.1-8B decode step: 32 query heads, 8 kv heads, 8192 cached tokens
    wq = synth.decode_attn_qk(hq=32, hkv=8, tq=1, tk=8192, dh=128)
    check_qk(wq.tensors["Q"], wq.tensors["K"], 0.5, dev, TOL_BF16)
    wp = synth.attn_pv(h=32, hkv=8, tq=1, tk=8192, dv=128, rho=0.5, with_logits=True)
    check_pv(wp.tensors["P"], wp.tensors["V"], 0.5, dev, TOL_BF16)
    # PV on the energies the softmax pass emits: the GEMV ranks each head's
    # 8192 keys itself (32 keys per thread); rho = 1 writes identity lists
    P, E = check_softmax_energy(wp.tensors["L"], dev)
    Vt = wp.tensors["V"]
    for rho in (0.5, 1.0):
        idx, Og = rmm.pv_energy(P, Vt.to(dev), E, rho)
        torch.cuda.synchronize()
        Pc, Vc = f32(P), f32(Vt)
        idx_o, O_o = O.pv_given_energy(Pc, Vc, f32(E), rho)
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        assert_close(f32(Og), O_o, pv_envelope(Pc, Vc, idx_o), TOL_BF16, "PV")


def check_softmax_select(L, rho, dev, scale=1.0):
    P, E, idx = rmm.softmax_select(L.to(dev), rho, scale)
    torch.cuda.synchronize()
    Pg, Eg = f32(P), f32(E)
    Po = O.softmax_rows(f32(L), scale)
    assert rel_fro(Pg, Po) <= 1e-6
    assert np.max(np.abs(Pg - Po)) <= 1e-6 * np.max(Po)
    Eo = np.stack([O.col_energy(Pg[h]) for h in range(Pg.shape[0])])
    assert rel_fro(Eg, Eo) <= 1e-5
    # the lists are the selection on the energies the call wrote
    zero_v = np.zeros((Pg.shape[0], Pg.shape[2], 1))
    idx_o, _ = O.pv_given_energy(Pg, zero_v, Eg, rho)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    return P, E, idx


@pytest.mark.parametrize("h,tq,tk,rho", [(32, 1, 8192, 0.5), (8, 1, 1000, 0.3), (8, 2, 3000, 0.7),
                                         (16, 4, 2048, 1.0), (4, 96, 1024, 0.5), (2, 40, 300, 0.2)])
def test_softmax_select(dev, h, tq, tk, rho):
    # one workgroup per head ranks inside the softmax pass (8, 16 and 32 keys
    # per thread, 1 to 4 query rows); longer query blocks run the softmax
    # pass and then TopK over its energies
    w = synth.attn_pv(h=h, hkv=1, tq=tq, tk=tk, dv=8, rho=min(rho, 0.9), with_logits=True)
    print(f"softmax_select h={h} tq={tq} tk={tk} rho={rho}", flush=True)
    check_softmax_select(w.tensors["L"], rho, dev, scale=0.5)


@pytest.mark.parametrize("h,hkv,tq,tk,dv,vdt", [(32, 8, 1, 8192, 128, torch.bfloat16),
                                                (8, 2, 4, 1000, 64, torch.bfloat16),
                                                (4, 2, 96, 1024, 64, torch.bfloat16),
                                                (4, 1, 20, 300, 24, torch.float32)])
def test_pv_idx(dev, h, hkv, tq, tk, dv, vdt):
    # PV over given per-head lists: the GEMV per head (tq <= 16), the packed
    # product, and fp32 V (vector-ALU product); lists unsorted, with repeats
    # and entries outside [0, tk)
    w = synth.attn_pv(h=h, hkv=hkv, tq=tq, tk=tk, dv=dv, rho=0.5)
    P, V = w.tensors["P"], w.tensors["V"].to(vdt)
    k = tk // 2
    idx = np.stack([_given_idx(tk, k, seed=100 + i) for i in range(h)])
    print(f"pv_idx h={h} tq={tq} tk={tk} dv={dv} {vdt}", flush=True)
    Og = rmm.pv_idx(P.to(dev), V.to(dev), torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    Pc, Vc = f32(P), f32(V)
    g = h // hkv
    ref = np.stack([O.matmul_given(Pc[i], Vc[i // g], idx[i]) for i in range(h)])
    env = np.stack([envelope(Pc[i], Vc[i // g], idx[i]) for i in range(h)])
    assert_close(f32(Og), ref, env, TOL_FP32 if vdt == torch.float32 else TOL_BF16, "PV over given lists")


def test_decode_attention_softmax_select_then_pv_idx(dev):
    # the ranking inside the softmax pass and the TopK launch of
    # rmm_pv_energy, on the same P and energies, keep the same lists, and the
    # PV over those lists is the same GEMV: bit for bit
    w = synth.attn_pv(h=32, hkv=8, tq=1, tk=8192, dv=128, rho=0.5, with_logits=True)
    Ld, Vd = w.tensors["L"].to(dev), w.tensors["V"].to(dev)
    P1, E1, idx1 = check_softmax_select(w.tensors["L"], 0.5, dev, scale=128 ** -0.5)
    O1 = rmm.pv_idx(P1, Vd, idx1)
    idx2, O2 = rmm.pv_energy(P1, Vd, E1, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(O1.view(torch.int32), O2.view(torch.int32))
    Pc, Vc = f32(P1), f32(w.tensors["V"])
    idx_o, O_o = O.pv_given_energy(Pc, Vc, f32(E1), 0.5)
    assert_close(f32(O1), O_o, pv_envelope(Pc, Vc, idx_o), TOL_BF16, "PV")


# ----------------------------- full sizes -----------------------------------

def test_full_mlp_down(dev):
    w = synth.mlp_down()
    A, B = w.tensors["A"], w.tensors["B"]
    rows = tile_rows(A.shape[0])
    for rho in (0.9, 0.7, 0.5, 1.0):
        print(f"mlp_down 4096x14336x4096 rho={rho}", flush=True)
        check_matmul(A, B, rho, dev, TOL_BF16, rows=rows)


def test_full_decode_qkv(dev):
    w = synth.decode_qkv()
    for rho in (0.8, 1.0):
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)


@pytest.mark.parametrize("rho", [0.5, 1.0])
def test_linear_last_wave_split(dev, rho):
    # 500 x 34776 output: 2 x 136 tiles of 256 x 256 would leave a last wave
    # of 16 tiles, so the first 32768 columns run as two whole waves of
    # 256 x 256 tiles and the last 2008 (a ragged band) as 128 x 128 tiles in
    # a second launch; every row and column compared, fp32 and bf16 output,
    # bf16 and int8 weights
    w = synth.mlp_down(n=500, d=448, m=34776, rhos=(0.5,))
    check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16)
    check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16, out_dtype=torch.bfloat16)
    w8 = synth.w8_projection(n=500, d=448, m=34776, rho=rho, name="w8_last_wave")
    check_matmul_w8(w8, rho, dev, TOL_BF16)


def test_full_mlp_up(dev):
    w = synth.mlp_up()
    rows = tile_rows(2048)[::2]
    for rho in (0.8, 1.0):
        print(f"mlp_up 2048x8192x28672 rho={rho}", flush=True)
        check_matmul(w.tensors["A"], w.tensors["B"], rho, dev, TOL_BF16, rows=rows)


@pytest.mark.parametrize("rho,out_dtype", [(0.5, torch.float32), (0.9, torch.float32), (0.5, torch.bfloat16)])
def test_qk_many_tiles_ragged(dev, rho, out_dtype):
    # 32 heads x 1100 x 1100: 800 score tiles of 256 x 256, so the persistent
    # product walks 3 or 4 tiles per workgroup across heads, with ragged
    # last tile rows and columns (1100 = 4 x 256 + 76); one K step (rho 0.5:
    # 64 kept features) or two (rho 0.9: 116 kept, padded to 128); fp32
    # output (whole tiles stored without a per-element test) and bf16
    w = synth.gqa_qk(hq=32, hkv=8, t=1100, dh=128)
    check_qk(w.tensors["Q"], w.tensors["K"], rho, dev, TOL_BF16, out_dtype=out_dtype)


@pytest.mark.parametrize("rho,out_dtype", [(0.5, torch.float32), (1.0, torch.bfloat16)])
def test_qk_causal_many_tiles_ragged(dev, rho, out_dtype):
    # the same 800 tiles with the causal mask: tiles wholly above the
    # diagonal stored as -inf without a test per element, diagonal and
    # ragged tiles element by element; then 900 queries at the end of 1100
    # keys (the diagonal shifted by 200; 640 tiles)
    w = synth.gqa_qk(hq=32, hkv=8, t=1100, dh=128)
    check_qk_causal(w.tensors["Q"], w.tensors["K"], rho, dev, TOL_BF16, out_dtype=out_dtype)
    check_qk_causal(w.tensors["Q"][:, -900:, :].contiguous(), w.tensors["K"], rho, dev, TOL_BF16)


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
        Qf, Kf = f32(Q), f32(K)
        i_o, S_o = O.qk(Qf, Kf, rho, heads=hs)
        assert_close(f32(S[torch.as_tensor(hs, device=S.device)]), S_o, qk_envelope(Qf, Kf, i_o, hs), TOL_BF16,
                     "scores")
        del S


def test_full_attn_pv_with_producer(dev):
    w = synth.attn_pv(with_logits=True)
    heads = [0, 9, 37, 63]
    P, E = check_softmax_energy(w.tensors["L"], dev, heads=heads)
    idx, Og = rmm.pv_energy(P, w.tensors["V"].to(dev), E, 0.5)
    torch.cuda.synchronize()
    # the oracle selects on the energies of the P the kernel wrote and forms
    # the product over those keys (sampled heads)
    Pc = f32(P)
    Eo = np.stack([O.col_energy(Pc[h]) if h in heads else np.zeros(Pc.shape[2]) for h in range(Pc.shape[0])])
    Vc = f32(w.tensors["V"])
    idx_o, O_o = O.pv_given_energy(Pc, Vc, Eo, 0.5, heads=heads)
    np.testing.assert_array_equal(idx.cpu().numpy()[heads], idx_o)
    assert_close(f32(Og[torch.as_tensor(heads, device=Og.device)]), O_o, pv_envelope(Pc, Vc, idx_o, heads),
                 TOL_BF16, "PV")


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
        Vn = f32(V)
        i_o, O_o = O.pv(Pn, Vn, rho, heads=hs)
        assert_close(f32(Og[torch.as_tensor(hs, device=Og.device)]), O_o, pv_envelope(Pn, Vn, i_o, hs), TOL_BF16,
                     "PV")
