"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/rmm.h declares, and
reject bad arguments before it touches the HIP runtime.  Only argument
errors are exercised here: a call that passes validation would launch work.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from input_adaptive_reduced_colnorm_amd import rmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmm.h")

OK, NULL, RHO, SHAPE, DTYPE, ALIGN, WS, HIP, ALIAS = range(9)
FP32, BF16 = 0, 1
FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rmm_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return rmm.lib()


def test_library_exports_every_declared_function(L):
    names = header_functions()
    assert {"rmm_k", "rmm_select", "rmm_matmul", "rmm_qk", "rmm_pv"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", rmm._LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(rmm_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        assert n in rmm.SIGNATURES, f"binding lacks {n}"
        getattr(L, n)


def test_k_rule_through_the_abi(L):
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "k_rule.json")))["cases"]
    for c in cases:
        assert L.rmm_k(c["rho"], c["d"]) == c["k"], c
    for bad in (0.0, -0.5, 1.0000001, math.nan, math.inf):
        assert L.rmm_k(bad, 10) == -1
    assert L.rmm_k(0.5, 0) == -1


def test_status_strings(L):
    for s in range(9):
        assert L.rmm_status_str(s).decode().startswith("RMM_")
    assert L.rmm_status_str(99) == b"unknown rmm status"


def _matmul(L, A=FAKE, B=FAKE + (1 << 30), dt=BF16, n=64, d=128, m=64, lda=128, ldb=64, rho=0.5,
            idx=FAKE + (2 << 30), Y=FAKE + (3 << 30), ydt=FP32, ldy=64, ws=FAKE + (4 << 30), wsb=1 << 30):
    return L.rmm_matmul(A, B, dt, n, d, m, lda, ldb, rho, idx, Y, ydt, ldy, ws, wsb, None)


def test_matmul_rejects_bad_arguments(L):
    assert _matmul(L, A=None) == NULL
    assert _matmul(L, B=None) == NULL
    assert _matmul(L, idx=None) == NULL
    assert _matmul(L, Y=None) == NULL
    for r in (0.0, -0.1, 1.5, math.nan, math.inf):
        assert _matmul(L, rho=r) == RHO
    assert _matmul(L, dt=7) == DTYPE
    assert _matmul(L, ydt=-1) == DTYPE
    assert _matmul(L, n=0) == SHAPE          # empty input
    assert _matmul(L, d=0) == SHAPE
    assert _matmul(L, m=-3) == SHAPE
    assert _matmul(L, lda=100) == SHAPE      # lda < d
    assert _matmul(L, ldb=8) == SHAPE
    assert _matmul(L, ldy=8) == SHAPE
    assert _matmul(L, A=FAKE + 1) == ALIGN   # bf16 needs 2-byte alignment
    assert _matmul(L, ws=None) == WS
    assert _matmul(L, wsb=16) == WS
    assert _matmul(L, ws=FAKE + (4 << 30) + 8) == WS   # not 256-byte aligned
    assert _matmul(L, Y=FAKE) == ALIAS       # output on top of A
    assert _matmul(L, idx=FAKE + (1 << 30)) == ALIAS   # index output on top of B
    assert _matmul(L, ws=FAKE + (3 << 30)) == ALIAS    # workspace overlaps Y


def test_matmul_size_limits(L):
    # dimensions reach 2^31 - 1 at most; a bf16 operand the matrix-core
    # loaders address must stay below 2 GiB (32-bit byte offsets)
    far = dict(B=FAKE + (1 << 40), idx=FAKE + (2 << 40), Y=FAKE + (3 << 40), ws=FAKE + (4 << 40), wsb=1 << 40)
    assert _matmul(L, d=1 << 31, lda=1 << 31, **far) == SHAPE
    assert _matmul(L, m=1 << 31, ldb=1 << 31, ldy=1 << 31, **far) == SHAPE
    assert _matmul(L, d=32768, lda=32768, m=32768, ldb=32768, ldy=32768, **far) == SHAPE   # B is 2 GiB


def test_matmul_workspace_covers_an_element_aligned_dense_a(L):
    # rho = 1 reads a 16-byte aligned A in place, but the query does not
    # know the pointer: an A that is only 2-byte aligned (a column-offset
    # view) is packed, n x d bf16 plus the padded index list
    assert L.rmm_matmul_workspace(64, 128, 64, 128, BF16, 1.0) >= 64 * 128 * 2 + 128 * 4
    assert L.rmm_matmul_workspace(64, 128, 64, 128, BF16, 0.5) > 0
    assert L.rmm_matmul_workspace(0, 128, 64, 128, BF16, 0.5) == 0   # invalid shape


def test_qk_rejects_bad_arguments(L):
    base = dict(Q=FAKE, K=FAKE + (1 << 30), dt=BF16, hq=4, hkv=2, tq=16, tk=16, dh=64, qhs=1024, qts=64,
                khs=1024, kts=64, rho=0.5, idx=FAKE + (2 << 30), S=FAKE + (3 << 30), sdt=FP32,
                ws=FAKE + (4 << 30), wsb=1 << 30)

    def call(fn=L.rmm_qk, **kw):
        a = dict(base, **kw)
        return fn(a["Q"], a["K"], a["dt"], a["hq"], a["hkv"], a["tq"], a["tk"], a["dh"], a["qhs"], a["qts"],
                  a["khs"], a["kts"], a["rho"], a["idx"], a["S"], a["sdt"], a["ws"], a["wsb"], None)

    for fn in (L.rmm_qk, L.rmm_qk_causal):
        assert call(fn, Q=None) == NULL
        assert call(fn, rho=0.0) == RHO
        assert call(fn, hkv=3) == SHAPE              # hq % hkv != 0
        assert call(fn, tq=0) == SHAPE
        assert call(fn, qts=32) == SHAPE             # row stride shorter than the head dim
        assert call(fn, dt=5) == DTYPE
        assert call(fn, wsb=0) == WS
        assert call(fn, S=FAKE + (1 << 30)) == ALIAS
    # causal scores: the queries are the last tq of the tk positions
    assert call(L.rmm_qk_causal, tq=17, qhs=17 * 64) == SHAPE


def test_pv_rejects_bad_arguments(L):
    base = dict(P=FAKE, pdt=FP32, V=FAKE + (1 << 30), vdt=BF16, h=4, hkv=2, tq=8, tk=64, dv=16, phs=512, pts=64,
                vhs=1024, vts=16, rho=0.5, idx=FAKE + (2 << 30), O=FAKE + (3 << 30), odt=FP32,
                ws=FAKE + (4 << 30), wsb=1 << 30)

    def call(**kw):
        a = dict(base, **kw)
        return L.rmm_pv(a["P"], a["pdt"], a["V"], a["vdt"], a["h"], a["hkv"], a["tq"], a["tk"], a["dv"], a["phs"],
                        a["pts"], a["vhs"], a["vts"], a["rho"], a["idx"], a["O"], a["odt"], a["ws"], a["wsb"], None)

    assert call(V=None) == NULL
    assert call(rho=2.0) == RHO
    assert call(h=6, hkv=4) == SHAPE
    assert call(pts=32) == SHAPE             # P row shorter than tk
    assert call(vdt=3) == DTYPE
    assert call(P=FAKE + 2) == ALIGN         # fp32 needs 4-byte alignment
    assert call(ws=None) == WS
    assert call(O=FAKE) == ALIAS


def test_select_rejects_bad_arguments(L):
    def call(A=FAKE, dt=FP32, n=8, d=32, lda=32, rho=0.5, idx=FAKE + (1 << 30), sc=None, ws=FAKE + (2 << 30),
             wsb=1 << 30):
        return L.rmm_select(A, dt, n, d, lda, rho, idx, sc, ws, wsb, None)

    assert call(A=None) == NULL
    assert call(rho=math.nan) == RHO
    assert call(lda=16) == SHAPE
    assert call(dt=2) == DTYPE
    assert call(wsb=4) == WS
    assert call(idx=FAKE) == ALIAS
    assert call(sc=FAKE + 4) == ALIAS


def test_timed_variants_check_events_then_arguments(L):
    """The stage-timed entry points need five event handles, then validate
    exactly like the plain calls (fake handles are never touched because
    validation fails before the first event is recorded)."""
    ev_ok = (ctypes.c_void_p * 5)(*([FAKE + (5 << 30)] * 5))
    ev_hole = (ctypes.c_void_p * 5)(FAKE, FAKE, None, FAKE, FAKE)
    mm = [FAKE, FAKE + (1 << 30), BF16, 512, 1024, 256, 1024, 256, 0.5, FAKE + (2 << 30), FAKE + (3 << 30), FP32, 256,
          FAKE + (4 << 30), 1 << 30, None]
    assert L.rmm_matmul_timed(*mm, None) == NULL
    assert L.rmm_matmul_timed(*mm, ev_hole) == NULL
    bad = list(mm)
    bad[8] = 0.0
    assert L.rmm_matmul_timed(*bad, ev_ok) == RHO
    qk = [FAKE, FAKE + (1 << 30), BF16, 4, 2, 16, 16, 64, 1024, 64, 1024, 64, 0.5, FAKE + (2 << 30),
          FAKE + (3 << 30), FP32, FAKE + (4 << 30), 1 << 30, None]
    assert L.rmm_qk_timed(*qk, None) == NULL
    assert L.rmm_qk_timed(*qk, ev_hole) == NULL
    bad = list(qk)
    bad[4] = 3                                # hq % hkv != 0
    assert L.rmm_qk_timed(*bad, ev_ok) == SHAPE
    pv = [FAKE, FP32, FAKE + (1 << 30), BF16, 4, 2, 8, 64, 16, 512, 64, 1024, 16, 0.5, FAKE + (2 << 30),
          FAKE + (3 << 30), FP32, FAKE + (4 << 30), 1 << 30, None]
    assert L.rmm_pv_timed(*pv, None) == NULL
    assert L.rmm_pv_timed(*pv, ev_hole) == NULL
    bad = list(pv)
    bad[3] = 9                                # unknown V dtype
    assert L.rmm_pv_timed(*bad, ev_ok) == DTYPE


def test_library_resolves_every_kernel_launch():
    """Each kernel the library launches must have its host launch stub in the
    library itself (a missing stub would only fail at the first call)."""
    path = rmm._LIB_PATH
    out = subprocess.run(["nm", "-u", "-C", path], capture_output=True, text=True, check=True).stdout
    missing = [l.strip() for l in out.splitlines() if "__device_stub__" in l]
    assert not missing, missing


def test_matmul_w8_rejects_bad_arguments(L):
    def call(A=FAKE, adt=BF16, Bq=FAKE + (1 << 30), sc=FAKE + (5 << 30), n=64, d=128, m=64, lda=128, ldb=64, rho=0.5,
             idx=FAKE + (2 << 30), Y=FAKE + (3 << 30), ydt=FP32, ldy=64, ws=FAKE + (4 << 30), wsb=1 << 30):
        return L.rmm_matmul_w8(A, adt, Bq, sc, n, d, m, lda, ldb, rho, idx, Y, ydt, ldy, ws, wsb, None)

    assert call(Bq=None) == NULL
    assert call(sc=None) == NULL
    assert call(rho=0.0) == RHO
    assert call(adt=FP32) == DTYPE           # int8 weights take bf16 activations
    assert call(m=60, ldb=64, ldy=64) == SHAPE   # columns not a multiple of 8
    assert call(ldb=68) == SHAPE             # row stride not a multiple of 8
    assert call(ldb=32) == SHAPE             # ldb < m
    assert call(Bq=FAKE + (1 << 30) + 4) == ALIGN   # 8-byte loads
    assert call(sc=FAKE + (5 << 30) + 2) == ALIGN
    assert call(ws=None) == WS
    assert call(Y=FAKE + (1 << 30)) == ALIAS     # output on top of the weights
    assert call(idx=FAKE + (5 << 30)) == ALIAS   # index output on top of the scales
    assert L.rmm_matmul_w8_workspace(64, 128, 64, 128, 1.0) >= 0
    assert L.rmm_matmul_w8_workspace(64, 128, 64, 128, 0.5) > 0
    assert L.rmm_matmul_w8_workspace(64, 128, 64, 100, 0.5) == 0   # lda < d
    assert L.rmm_matmul_w8_timed(FAKE, BF16, FAKE + (1 << 30), FAKE + (5 << 30), 64, 128, 64, 128, 64, 0.5,
                                 FAKE + (2 << 30), FAKE + (3 << 30), FP32, 64, None, 0, None, None) == NULL


def test_matmul_idx_rejects_bad_arguments(L):
    def call(A=FAKE, B=FAKE + (1 << 30), dt=BF16, n=64, d=128, m=64, lda=128, ldb=64, idx=FAKE + (2 << 30), k=32,
             Y=FAKE + (3 << 30), ydt=FP32, ldy=64, ws=FAKE + (4 << 30), wsb=1 << 30):
        return L.rmm_matmul_idx(A, B, dt, n, d, m, lda, ldb, idx, k, Y, ydt, ldy, ws, wsb, None)

    assert call(idx=None) == NULL
    assert call(dt=4) == DTYPE
    assert call(k=0) == SHAPE                # empty index list
    assert call(lda=64) == SHAPE
    assert call(ws=None) == WS               # the padded list always needs workspace
    assert call(Y=FAKE + 64) == ALIAS
    assert call(ws=FAKE + (1 << 30) + 256) == ALIAS
    assert L.rmm_matmul_idx_workspace(64, 32, 64, BF16) > 0
    assert L.rmm_matmul_idx_workspace(64, 0, 64, BF16) == 0


def test_softmax_energy_and_pv_energy_reject_bad_arguments(L):
    def sm(Lp=FAKE, scale=1.0, h=4, tq=16, tk=512, lhs=8192, lts=512, P=FAKE + (1 << 30), phs=8192, pts=512,
           E=FAKE + (2 << 30), ws=FAKE + (3 << 30), wsb=1 << 30):
        return L.rmm_softmax_energy(Lp, scale, h, tq, tk, lhs, lts, P, phs, pts, E, ws, wsb, None)

    assert sm(E=None) == NULL
    assert sm(scale=0.0) == SHAPE
    assert sm(scale=math.inf) == SHAPE
    assert sm(tk=20000) == SHAPE             # more keys than one row of registers holds
    assert sm(lts=100) == SHAPE
    assert sm(P=FAKE + 2) == ALIGN
    assert sm(wsb=4) == WS
    assert sm(P=FAKE + 4096) == ALIAS        # P on top of the logits
    assert L.rmm_softmax_energy_workspace(4, 16, 512) > 0

    def pe(E=FAKE + (5 << 30), rho=0.5, h=4, hkv=2):
        return L.rmm_pv_energy(FAKE, FP32, FAKE + (1 << 30), BF16, E, h, hkv, 8, 64, 16, 512, 64, 1024, 16, rho,
                               FAKE + (2 << 30), FAKE + (3 << 30), FP32, FAKE + (4 << 30), 1 << 30, None)

    assert pe(E=None) == NULL
    assert pe(rho=0.0) == RHO
    assert pe(h=6, hkv=4) == SHAPE
    assert pe(E=FAKE + (2 << 30)) == ALIAS   # energies on top of the index output


def test_softmax_select_and_pv_idx_reject_bad_arguments(L):
    def ss(Lp=FAKE, scale=1.0, h=4, tq=16, tk=512, lhs=8192, lts=512, P=FAKE + (1 << 30), phs=8192, pts=512,
           E=FAKE + (2 << 30), rho=0.5, idx=FAKE + (4 << 30), ws=FAKE + (3 << 30), wsb=1 << 30):
        return L.rmm_softmax_select(Lp, scale, h, tq, tk, lhs, lts, P, phs, pts, E, rho, idx, ws, wsb, None)

    assert ss(idx=None) == NULL
    assert ss(rho=0.0) == RHO
    assert ss(rho=1.5) == RHO
    assert ss(scale=-1.0) == SHAPE
    assert ss(tk=20000) == SHAPE
    assert ss(idx=FAKE + (4 << 30) + 2) == ALIGN
    assert ss(wsb=4) == WS                   # 16 rows of 4 heads: the separate TopK path needs scratch
    assert ss(idx=FAKE + (2 << 30) + 64) == ALIAS   # the lists on top of the energies
    # decode-shaped (one workgroup per head): no workspace at all
    assert L.rmm_softmax_select_workspace(4, 1, 512) == 0

    def pi(P=FAKE, pdt=FP32, V=FAKE + (1 << 30), vdt=BF16, idx=FAKE + (2 << 30), k=32, h=4, hkv=2, tq=8, tk=64,
           dv=16, O=FAKE + (3 << 30), ws=FAKE + (4 << 30), wsb=1 << 30):
        return L.rmm_pv_idx(P, pdt, V, vdt, idx, k, h, hkv, tq, tk, dv, 512, 64, 1024, 16, O, FP32, ws, wsb, None)

    assert pi(idx=None) == NULL
    assert pi(vdt=5) == DTYPE
    assert pi(k=0) == SHAPE
    assert pi(h=6, hkv=4) == SHAPE
    assert pi(idx=FAKE + (2 << 30) + 1) == ALIGN
    assert pi(ws=None) == WS                 # the padded lists always need workspace
    assert pi(O=FAKE + (2 << 30)) == ALIAS   # output on top of the lists
    assert L.rmm_pv_idx_workspace(4, 8, 32, 16, BF16) > 0


def test_generic_workspace_bound_covers_every_per_call_query(L):
    """rmm_workspace_bytes(op, ...) is at least the per-call query for every
    rho, dtype and size within its arguments' bounds."""
    rhos = [1e-3, 0.05, 0.3, 0.5, 0.7, 0.8, 0.9, 0.999, 1.0]
    for n, d, m in [(8, 4096, 6144), (16, 1000, 264), (17, 100, 48), (4096, 14336, 4096), (300, 64, 8),
                    (1, 20000, 8), (2048, 8192, 28672)]:
        for dt in (FP32, BF16):
            bs = L.rmm_workspace_bytes(0, n, d, 0)
            bm = L.rmm_workspace_bytes(1, n, d, m)
            bw = L.rmm_workspace_bytes(4, n, d, m)
            for lda in (d, d + 1, d + 8):
                for rho in rhos:
                    assert bm >= L.rmm_matmul_workspace(n, d, m, lda, dt, rho), (n, d, m, lda, dt, rho)
                    assert bw >= L.rmm_matmul_w8_workspace(n, d, m, lda, rho), (n, d, m, lda, rho)
            assert bs >= L.rmm_select_workspace(n, d, dt)
            for k in (1, d // 2, d, 3 * d):
                bi = L.rmm_workspace_bytes(5, n, k, m)
                assert bi >= L.rmm_matmul_idx_workspace(n, k, m, dt), (n, k, m, dt)
    for hq, dh, tq, tk in [(32, 128, 4096, 4096), (8, 40, 45, 45), (4, 256, 130, 130), (8, 128, 1, 1000),
                           (4, 64, 200, 520)]:
        bq = L.rmm_workspace_bytes(2, hq, dh, max(tq, tk))
        for dt in (FP32, BF16):
            for rho in rhos:
                assert bq >= L.rmm_qk_workspace(hq, tq, tk, dh, dt, rho), (hq, tq, tk, dh, dt, rho)
    for h, tq, tk, dv in [(64, 512, 8192, 128), (32, 1, 8192, 128), (4, 16, 512, 64), (8, 4, 1000, 128),
                          (2, 40, 300, 24), (4, 96, 1024, 64)]:
        bp = L.rmm_workspace_bytes(3, h, tk, max(tq, dv))
        be = L.rmm_workspace_bytes(7, h, tk, max(tq, dv))
        for pdt in (FP32, BF16):
            for vdt in (FP32, BF16):
                for rho in rhos:
                    assert bp >= L.rmm_pv_workspace(h, tq, tk, dv, pdt, vdt, rho), (h, tq, tk, dv, pdt, vdt, rho)
                    assert be >= L.rmm_pv_energy_workspace(h, tq, tk, dv, pdt, vdt, rho)
        if tk <= 8192:
            assert L.rmm_workspace_bytes(6, h, tk, tq) == L.rmm_softmax_energy_workspace(h, tq, tk)
            assert L.rmm_workspace_bytes(8, h, tk, tq) == L.rmm_softmax_select_workspace(h, tq, tk)
        for k in (1, tk // 2, tk, 2 * tk):
            bi = L.rmm_workspace_bytes(9, h, k, max(tq, dv))
            for vdt in (FP32, BF16):
                assert bi >= L.rmm_pv_idx_workspace(h, tq, k, dv, vdt), (h, tq, k, dv, vdt)
    # one workgroup per head (decode) ranks inside the softmax pass: no scratch
    assert L.rmm_softmax_select_workspace(32, 1, 8192) == 0
    assert L.rmm_softmax_select_workspace(64, 512, 8192) > 0
    # unknown op and bad sizes
    assert L.rmm_workspace_bytes(99, 8, 8, 8) == 0
    assert L.rmm_workspace_bytes(1, 0, 8, 8) == 0
    assert L.rmm_workspace_bytes(1, 8, -1, 8) == 0


def test_noalloc_matmul_rejects_bad_arguments_before_touching_the_device(L):
    def call(A=FAKE, B=FAKE + (1 << 30), dt=BF16, n=64, d=128, m=64, lda=128, ldb=64, rho=0.5,
             idx=FAKE + (2 << 30), Y=FAKE + (3 << 30), ydt=FP32, ldy=64):
        return L.rmm_matmul_noalloc(A, B, dt, n, d, m, lda, ldb, rho, idx, Y, ydt, ldy, None)
    assert call(A=None) == NULL
    assert call(rho=0.0) == RHO
    assert call(dt=7) == DTYPE
    assert call(lda=100) == SHAPE
    assert call(A=FAKE + 1) == ALIGN
    assert call(Y=FAKE + 16) == ALIAS
    # more scratch than the library's 32 MiB array: the packed A alone is
    # 2 * 4096 * 12928 bytes at rho = 0.9
    big = dict(B=FAKE + (1 << 40), idx=FAKE + (2 << 40), Y=FAKE + (3 << 40))
    assert call(n=4096, d=14336, m=256, lda=14336, ldb=256, ldy=256, rho=0.9, **big) == WS
