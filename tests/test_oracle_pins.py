"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these re-derive the oracle's own formula: they use hand-worked
values, exact rational arithmetic, pure-Python loops, brute force over all
subsets, closed forms and invariants.  Each pin is written as a checker that
takes an oracle-like namespace, so planted mistakes (mutants at the bottom of
this file) can be shown to fail at least one pin.
"""

import itertools
import json
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import rmm_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _loop_matmul(A, B):
    """Pure-Python triple loop with exactly rounded sums (math.fsum)."""
    n, d = len(A), len(A[0])
    m = len(B[0])
    return [[math.fsum(float(A[i][t]) * float(B[t][j]) for t in range(d)) for j in range(m)]
            for i in range(n)]


# --------------------------------------------------------------------------
# pin checkers (return None when the pin holds, else a message)
# --------------------------------------------------------------------------

def pin_k_rule(ns):
    for c in _load("k_rule.json")["cases"]:
        k = ns.k_rule(c["rho"], c["d"])
        if k != c["k"]:
            return f"k_rule({c['rho']}, {c['d']}) = {k}, hand value {c['k']}"
    # exact decimal arithmetic on many awkward products
    for num in range(1, 101):
        rho_s = f"{num / 100:.2f}"
        for d in (1, 3, 7, 10, 100, 128, 999, 4096, 14336):
            want = math.ceil(Fraction(rho_s) * d)
            want = max(1, min(d, want))
            got = ns.k_rule(float(rho_s), d)
            if got != want:
                return f"k_rule({rho_s}, {d}) = {got}, exact decimal ceil {want}"
    return None


def pin_worked_example(ns):
    g = _load("worked_example.json")
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    if not np.array_equal(ns.col_energy(A), np.array(g["col_energy"], dtype=np.float64)):
        return "column energies differ from the hand values"
    for c in g["cases"]:
        idx, Y = ns.matmul(A, B, c["rho"])
        if list(np.asarray(idx)) != c["idx"]:
            return f"rho={c['rho']}: idx {list(idx)} != hand {c['idx']}"
        if not np.array_equal(np.asarray(Y), np.array(c["Y"], dtype=np.float64)):
            return f"rho={c['rho']}: Y differs from the hand value"
        err = float(np.linalg.norm(A @ B - Y))
        if abs(err - c["err_fro"]) > 1e-12 * max(1.0, c["err_fro"]):
            return f"rho={c['rho']}: error {err} != hand {c['err_fro']}"
        bnd = ns.error_bound(A, B, idx)
        if abs(bnd - c["bound"]) > 1e-12 * max(1.0, c["bound"]):
            return f"rho={c['rho']}: bound {bnd} != hand {c['bound']}"
    return None


def pin_dense_loop(ns):
    """rho = 1 keeps every index and gives the unreduced product; `dense`
    (the unreduced product on its own) equals the same exactly rounded
    triple loop, on a non-square case so that a transposed or truncated
    operand cannot pass."""
    r = np.random.default_rng(7)
    A = r.standard_normal((5, 7))
    B = r.standard_normal((7, 3))
    idx, Y = ns.matmul(A, B, 1.0)
    if list(np.asarray(idx)) != list(range(7)):
        return "rho=1 must keep every index"
    ref = np.array(_loop_matmul(A.tolist(), B.tolist()))
    if np.max(np.abs(np.asarray(Y) - ref)) > 1e-12 * np.max(np.abs(ref)):
        return "rho=1 product differs from the triple loop"
    # dense on bf16-representable values (float32 storage), the way the
    # tests feed it: entries k / 64 with |k| < 256 are exact in bf16
    A2 = r.integers(-255, 256, size=(6, 11)).astype(np.float32) / np.float32(64)
    B2 = (r.standard_normal((11, 4)) * 1e3).astype(np.float32)
    D = np.asarray(ns.dense(A2, B2))
    if D.shape != (6, 4):
        return f"dense has shape {D.shape}, expected (6, 4)"
    ref2 = np.array(_loop_matmul(A2.tolist(), B2.tolist()))
    if np.max(np.abs(D - ref2)) > 1e-12 * np.max(np.abs(ref2)):
        return "dense differs from the triple loop"
    return None


def pin_reduced_loop(ns):
    """Reduced product equals the triple loop restricted to the kept set,
    where the kept set is recomputed by brute-force comparison of norms."""
    r = np.random.default_rng(11)
    A = r.integers(-4, 5, size=(4, 9)).astype(np.float64)
    B = r.standard_normal((9, 5))
    rho = 0.5
    idx, Y = ns.matmul(A, B, rho)
    k = 5
    # brute force: an index is kept iff fewer than k indices beat it, where
    # "beats" means a larger energy, or an equal energy and a lower index
    energy = [sum(float(A[i][j]) ** 2 for i in range(4)) for j in range(9)]
    keep = [j for j in range(9)
            if sum(1 for t in range(9) if energy[t] > energy[j] or (energy[t] == energy[j] and t < j)) < k]
    if list(np.asarray(idx)) != keep:
        return f"kept set {list(idx)} != brute force {keep}"
    ref = np.array(_loop_matmul(A[:, keep].tolist(), B[keep, :].tolist()))
    if np.max(np.abs(np.asarray(Y) - ref)) > 1e-12 * np.max(np.abs(ref)):
        return "reduced product differs from the loop over the kept set"
    return None


def pin_minimax_bruteforce(ns):
    """TopK by column norm maximises the kept norm (and energy) sum over all
    k-subsets, i.e. minimises the worst-case error over B with unit rows
    (the pages' minimax property); ties go to the lexicographically smallest
    maximiser."""
    r = np.random.default_rng(3)
    for trial in range(6):
        d, n = 12, 5
        A = r.integers(-3, 4, size=(n, d)).astype(np.float64)
        if trial % 2 == 1:
            A[:, 7] = A[:, 2]          # planted exact tie
            A[:, 9] = -A[:, 4]         # sign-flipped copy: same energy
        q = [int(sum(int(v) ** 2 for v in A[:, j])) for j in range(d)]
        for k in (1, 3, 6, 11):
            rho = k / d
            idx, _ = ns.matmul(A, np.eye(d), rho)
            idx = tuple(int(i) for i in np.asarray(idx))
            best_q = max(sum(q[j] for j in S) for S in itertools.combinations(range(d), k))
            maximisers = [S for S in itertools.combinations(range(d), k)
                          if sum(q[j] for j in S) == best_q]
            if sum(q[j] for j in idx) != best_q:
                return f"trial {trial} k={k}: kept energy is not maximal"
            if idx != min(maximisers):
                return f"trial {trial} k={k}: {idx} is not the lexicographically smallest maximiser"
            s = [math.sqrt(v) for v in q]
            best_s = max(math.fsum(s[j] for j in S) for S in itertools.combinations(range(d), k))
            if math.fsum(s[j] for j in idx) < best_s * (1 - 1e-12):
                return f"trial {trial} k={k}: kept norm sum is not maximal"
    return None


def pin_error_bound(ns):
    """||AB - A_I B_I||_F <= sum_{j not in I} ||A_j|| ||B_j|| on generated inputs."""
    cases = []
    w = synth.tiny_projection()
    cases.append((synth.stored64(w.tensors["A"]), synth.stored64(w.tensors["B"]), 0.5))
    w = synth.mlp_down(n=64, d=512, m=96)
    for rho in w.rhos:
        cases.append((synth.stored64(w.tensors["A"]), synth.stored64(w.tensors["B"]), rho))
    for A, B, rho in cases:
        idx, Y = ns.matmul(A, B, rho)
        err = float(np.linalg.norm(A @ B - np.asarray(Y)))
        bnd = ns.error_bound(A, B, idx)
        if not err <= bnd * (1 + 1e-12) + 1e-300:
            return f"error {err} exceeds bound {bnd} at rho={rho}"
    return None


def pin_worst_case(ns):
    """Orthonormal dropped rows of B attain error sqrt(sum dropped energy)."""
    r = np.random.default_rng(5)
    n, d, m = 10, 8, 6
    A = r.standard_normal((n, d))
    rho = 0.5
    idx, _ = ns.matmul(A, np.zeros((d, m)), rho)
    drop = [j for j in range(d) if j not in set(int(i) for i in np.asarray(idx))]
    Qm, _ = np.linalg.qr(r.standard_normal((m, m)))
    B = r.standard_normal((d, m))
    for t, j in enumerate(drop):
        B[j] = Qm[t]
    _, Y = ns.matmul(A, B, rho)
    err = float(np.linalg.norm(A @ B - np.asarray(Y)))
    want = math.sqrt(math.fsum(float(A[i, j]) ** 2 for i in range(n) for j in drop))
    if abs(err - want) > 1e-12 * want:
        return f"worst-case error {err} != closed form {want}"
    return None


def pin_ties(ns):
    # all columns identical: the first k are kept
    A = np.tile(np.array([[1.0], [2.0], [-2.0]]), (1, 10))
    idx, _ = ns.matmul(A, np.eye(10), 0.3)
    if list(np.asarray(idx)) != [0, 1, 2]:
        return f"identical columns: {list(idx)}"
    # zero columns are kept only when nothing else is left, lowest first
    A = np.zeros((2, 6))
    A[:, 4] = [1, 1]
    idx, _ = ns.matmul(A, np.eye(6), 0.5)
    if list(np.asarray(idx)) != [0, 1, 4]:
        return f"zero columns: {list(idx)}"
    # k = 1 is the first argmax
    A = np.array([[1.0, 3.0, -3.0, 2.0]])
    idx, _ = ns.matmul(A, np.eye(4), 0.25)
    if list(np.asarray(idx)) != [int(np.argmax(np.abs(A[0])))]:
        return f"k=1: {list(idx)}"
    return None


def pin_invariances(ns):
    r = np.random.default_rng(9)
    w = synth.mlp_down(n=32, d=256, m=40)
    A = synth.stored64(w.tensors["A"])
    B = synth.stored64(w.tensors["B"])
    rho = 0.7
    idx, Y = ns.matmul(A, B, rho)
    # scaling by a power of two is exact
    idx2, Y2 = ns.matmul(4.0 * A, B, rho)
    if not np.array_equal(np.asarray(idx2), np.asarray(idx)) or not np.array_equal(np.asarray(Y2), 4.0 * np.asarray(Y)):
        return "scaling A changed the selection or did not scale Y"
    # sign flips of columns (with the matching rows of B) change nothing
    sg = np.where(r.random(256) < 0.5, -1.0, 1.0)
    idx3, Y3 = ns.matmul(A * sg, B * sg[:, None], rho)
    if not np.array_equal(np.asarray(idx3), np.asarray(idx)) or np.max(np.abs(np.asarray(Y3) - np.asarray(Y))) > 1e-12 * np.max(np.abs(Y)):
        return "sign flips changed the result"
    # permuting columns of A with rows of B permutes I and keeps Y
    perm = r.permutation(256)
    idx4, Y4 = ns.matmul(A[:, perm], B[perm, :], rho)
    if sorted(int(perm[i]) for i in np.asarray(idx4)) != [int(i) for i in np.asarray(idx)]:
        return "permutation did not permute the kept set"
    if np.max(np.abs(np.asarray(Y4) - np.asarray(Y))) > 1e-12 * np.max(np.abs(Y)):
        return "permutation changed Y"
    return None


def pin_qk(ns):
    r = np.random.default_rng(13)
    hq, hkv, tq, tk, dh = 4, 2, 3, 5, 8
    Q = r.standard_normal((hq, tq, dh))
    K = r.standard_normal((hkv, tk, dh))
    idx, S = ns.qk(Q, K, 1.0)
    Kx = np.repeat(K, hq // hkv, axis=0)   # Llama-style repeat of K/V heads
    for h in range(hq):
        ref = np.array(_loop_matmul(Q[h].tolist(), Kx[h].T.tolist()))
        if np.max(np.abs(np.asarray(S[h]) - ref)) > 1e-12 * np.max(np.abs(ref)):
            return f"rho=1 QK^T head {h} differs from the triple loop"
    idx, S = ns.qk(Q, K, 0.5)
    idx_r, S_r = ns.qk(Q, Kx, 0.5)
    if not np.array_equal(np.asarray(idx), np.asarray(idx_r)) or np.max(np.abs(np.asarray(S) - np.asarray(S_r))) > 0:
        return "GQA gather differs from explicitly repeated K heads"
    for h in range(hq):
        q = np.sum(Q[h] ** 2, axis=0)
        kept = set(int(i) for i in np.asarray(idx[h]))
        if min(q[j] for j in kept) < max(q[j] for j in range(dh) if j not in kept):
            return f"head {h}: a dropped feature outranks a kept one"
        ref = np.array(_loop_matmul(Q[h][:, sorted(kept)].tolist(), Kx[h][:, sorted(kept)].T.tolist()))
        if np.max(np.abs(np.asarray(S[h]) - ref)) > 1e-12 * np.max(np.abs(ref)):
            return f"head {h}: reduced QK^T differs from the loop over kept features"
    return None


def pin_causal_qk(ns):
    """Causal scores: query row r of tq is position r + tk - tq of the key
    sequence, so its row must equal the unmasked scores against the keys up
    to that position, and its softmax must put zero weight on every later
    key.  The mask must leave the kept features unchanged, and a single
    query (decode) sees every key."""
    r = np.random.default_rng(29)
    hq, hkv, tq, tk, dh = 4, 2, 5, 9, 8
    Q = r.standard_normal((hq, tq, dh))
    K = r.standard_normal((hkv, tk, dh))
    idx, S = ns.qk(Q, K, 0.5)
    idx_c, S_c = ns.qk(Q, K, 0.5, causal=True)
    if not np.array_equal(np.asarray(idx), np.asarray(idx_c)):
        return "the causal mask changed the kept features"
    P_c = np.asarray(ns.softmax_rows(S_c))
    for row in range(tq):
        seen = row + tk - tq + 1
        _, S_p = ns.qk(Q, K[:, :seen, :], 0.5)
        if np.max(np.abs(np.asarray(S_c)[:, row, :seen] - np.asarray(S_p)[:, row, :])) > 0:
            return f"row {row}: visible scores differ from the scores against the first {seen} keys"
        P_p = np.asarray(ns.softmax_rows(S_p))[:, row, :]
        if np.max(np.abs(P_c[:, row, :seen] - P_p)) > 1e-15 or np.any(P_c[:, row, seen:] != 0.0):
            return f"row {row}: softmax weight on a key after the query position"
    _, S1 = ns.qk(Q[:, -1:, :], K, 0.5)
    _, S1c = ns.qk(Q[:, -1:, :], K, 0.5, causal=True)
    if not np.array_equal(np.asarray(S1), np.asarray(S1c)):
        return "a single causal query does not see every key"
    try:
        ns.qk(K[:, :, :], Q[:2, :3, :], 0.5, causal=True)
    except ValueError:
        return None
    return "causal scores accepted tq > tk"


def pin_pv(ns):
    r = np.random.default_rng(17)
    h, hkv, tq, tk, dv = 4, 1, 3, 10, 4
    L = r.standard_normal((h, tq, tk)) * 2
    P = np.exp(L) / np.exp(L).sum(axis=2, keepdims=True)
    V = r.standard_normal((hkv, tk, dv))
    idx, Ov = ns.pv(P, V, 1.0)
    for hh in range(h):
        ref = np.array(_loop_matmul(P[hh].tolist(), V[0].tolist()))
        if np.max(np.abs(np.asarray(Ov[hh]) - ref)) > 1e-12 * np.max(np.abs(ref)):
            return f"rho=1 PV head {hh} differs from the triple loop"
    Vx = np.repeat(V, h // hkv, axis=0)
    idx, Ov = ns.pv(P, V, 0.5)
    idx_r, O_r = ns.pv(P, Vx, 0.5)
    if not np.array_equal(np.asarray(idx), np.asarray(idx_r)) or np.max(np.abs(np.asarray(Ov) - np.asarray(O_r))) > 0:
        return "GQA gather differs from explicitly repeated V heads"
    for hh in range(h):
        q = np.sum(P[hh] ** 2, axis=0)
        kept = sorted(int(i) for i in np.asarray(idx[hh]))
        if min(q[kept]) < max(q[j] for j in range(tk) if j not in kept):
            return f"head {hh}: a dropped key outranks a kept one"
        ref = np.array(_loop_matmul(P[hh][:, kept].tolist(), V[0][kept, :].tolist()))
        if np.max(np.abs(np.asarray(Ov[hh]) - ref)) > 1e-12 * np.max(np.abs(ref)):
            return f"head {hh}: reduced PV differs from the loop over kept keys"
        err = float(np.linalg.norm(P[hh] @ V[0] - np.asarray(Ov[hh])))
        drop = [j for j in range(tk) if j not in kept]
        bnd = math.fsum(math.sqrt(q[j]) * float(np.linalg.norm(V[0][j])) for j in drop)
        if err > bnd * (1 + 1e-12):
            return f"head {hh}: PV error exceeds the bound"
    return None


def pin_given_index(ns):
    """The product over a given list against a pure-Python loop over the
    list's entries (any order, repeats, entries outside [0, d) skipped), and
    against the selected-set product when the list is the selection."""
    r = np.random.default_rng(77)
    A = r.integers(-4, 5, size=(5, 9)).astype(np.float64)
    B = r.integers(-3, 4, size=(9, 6)).astype(np.float64)
    for idx in ([4, 0, 7], [2, 2, 5], [-1, 3, 9, 100, 8], [8, 7, 6, 5, 4, 3, 2, 1, 0], [-3]):
        got = np.asarray(ns.matmul_given(A, B, np.asarray(idx, dtype=np.int32)))
        valid = [t for t in idx if 0 <= t < A.shape[1]]
        ref = [[math.fsum(A[i][t] * B[t][j] for t in valid) for j in range(B.shape[1])] for i in range(A.shape[0])]
        if got.shape != (5, 6) or np.max(np.abs(got - np.asarray(ref))) > 0:
            return f"given list {idx}: product differs from the loop over its valid entries"
    w = synth.mlp_down(n=24, d=40, m=12, rhos=(0.5,))
    A2, B2 = synth.stored64(w.tensors["A"]), synth.stored64(w.tensors["B"])
    I, Y = ns.matmul(A2, B2, 0.5)
    Yg = np.asarray(ns.matmul_given(A2, B2, np.asarray(I)[::-1].copy()))
    if np.max(np.abs(Yg - np.asarray(Y))) > 1e-12 * np.max(np.abs(Y)):
        return "the product over the selected list differs from the reduced product"
    return None


def pin_matmul_w8(ns):
    """int8 weights: with integer activations and power-of-two column scales
    every product and sum is exact, so the result must equal a pure-Python
    loop over the kept rows that multiplies each column by its own scale;
    negative weights near -128 catch a weight read as unsigned; the kept set
    is the float selection's."""
    r = np.random.default_rng(41)
    n, d, m = 6, 20, 7
    A = r.integers(-5, 6, size=(n, d)).astype(np.float64)
    A[:, 3] *= 9          # a clear top column
    Bq = r.integers(-128, 128, size=(d, m)).astype(np.int8)
    Bq[:, 0] = -128
    Bq[1, :] = -127
    scale = np.array([2.0 ** e for e in (-3, 1, 0, -7, 4, -1, 2)])
    for rho in (1.0, 0.55, 0.2):
        idx, Y = ns.matmul_w8(A, Bq, scale, rho)
        I, _ = ns.select(A, rho)
        if not np.array_equal(np.asarray(idx), np.asarray(I)):
            return f"rho {rho}: kept set differs from the float selection"
        ref = [[math.fsum(A[i][t] * int(Bq[t][c]) for t in I) * scale[c] for c in range(m)] for i in range(n)]
        if np.max(np.abs(np.asarray(Y) - np.asarray(ref))) > 0:
            return f"rho {rho}: int8 product differs from the per-column scaled loop"
    return None


def pin_softmax_energy(ns):
    """Row softmax against math.exp / fsum loops, shift invariance, and PV on
    supplied energies against PV scoring P itself."""
    r = np.random.default_rng(5)
    L = r.normal(0.0, 2.0, size=(2, 3, 7))
    P = np.asarray(ns.softmax_rows(L))
    for h in range(2):
        for i in range(3):
            row = [float(x) for x in L[h, i]]
            mx = max(row)
            ex = [math.exp(x - mx) for x in row]
            s = math.fsum(ex)
            if max(abs(P[h, i, j] - ex[j] / s) for j in range(7)) > 1e-15:
                return "softmax differs from the exp / fsum loop"
    if np.max(np.abs(np.asarray(ns.softmax_rows(L + 3.5)) - P)) > 1e-12:
        return "softmax changes when a row is shifted"
    if np.max(np.abs(np.asarray(ns.softmax_rows(L, 0.5)) - np.asarray(ns.softmax_rows(0.5 * L)))) > 1e-15:
        return "softmax of scaled logits differs from the softmax of the scaled values"
    w = synth.attn_pv(h=2, hkv=1, tq=12, tk=40, dv=8)
    P2, V2 = synth.stored64(w.tensors["P"]), synth.stored64(w.tensors["V"])
    E = np.stack([np.asarray(ns.col_energy(P2[h])) for h in range(2)])
    i1, o1 = ns.pv(P2, V2, 0.5)
    i2, o2 = ns.pv_given_energy(P2, V2, E, 0.5)
    if not np.array_equal(np.asarray(i1), np.asarray(i2)) or np.max(np.abs(np.asarray(o1) - np.asarray(o2))) > 0:
        return "PV on the column energies of P differs from PV scoring P"
    # other energies: the kept keys are exactly those of largest supplied energy
    E2 = -E
    i3, o3 = ns.pv_given_energy(P2, V2, E2, 0.5)
    for h in range(2):
        kept = set(int(j) for j in np.asarray(i3)[h])
        if min(E2[h][j] for j in kept) < max(E2[h][j] for j in range(40) if j not in kept):
            return "a dropped key has a larger supplied energy than a kept one"
        ref = np.array(_loop_matmul(P2[h][:, sorted(kept)].tolist(), V2[0][sorted(kept), :].tolist()))
        if np.max(np.abs(np.asarray(o3)[h] - ref)) > 1e-12 * np.max(np.abs(ref)):
            return "PV on supplied energies differs from the loop over its kept keys"
    return None


def pin_retained_energy(ns):
    """Brute force: the retained fraction equals the largest energy fraction
    any k-subset of columns keeps (TopK maximises the kept energy); ρ=1 keeps
    everything; integer columns make every sum exact."""
    r = np.random.default_rng(9)
    A = r.integers(-4, 5, size=(6, 10)).astype(np.float64)
    q = [math.fsum(float(A[i, j]) ** 2 for i in range(6)) for j in range(10)]
    tot = math.fsum(q)
    for rho in (0.1, 0.3, 0.5, 0.75, 0.95):
        k = ns.k_rule(rho, 10)
        best = max(math.fsum(q[j] for j in S) for S in itertools.combinations(range(10), k)) / tot
        got = ns.retained_energy(A, rho)
        if abs(got - best) > 1e-15:
            return f"rho {rho}: retained {got} but the best {k}-subset keeps {best}"
    if ns.retained_energy(A, 1.0) != 1.0:
        return "rho = 1 does not keep all the energy"
    return None


PINS = [pin_retained_energy, pin_k_rule, pin_worked_example, pin_dense_loop, pin_reduced_loop, pin_minimax_bruteforce,
        pin_error_bound, pin_worst_case, pin_ties, pin_invariances, pin_qk, pin_causal_qk, pin_pv, pin_given_index,
        pin_matmul_w8, pin_softmax_energy]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    msg = pin(O)
    assert msg is None, msg


def test_k_rule_rejects_bad_rho():
    for bad in (0.0, -0.1, 1.5, float("nan"), float("inf"), -float("inf")):
        with pytest.raises(ValueError):
            O.k_rule(bad, 10)
    with pytest.raises(ValueError):
        O.k_rule(0.5, 0)


# --------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# --------------------------------------------------------------------------

def _mutant(**over):
    ns = types.SimpleNamespace(**{k: getattr(O, k) for k in O.__all__})
    for k, v in over.items():
        setattr(ns, k, v)
    # rebuild the composite functions so they call the mutated pieces
    def select(A, rho, _ns=ns):
        A64 = np.asarray(A, dtype=np.float64)
        k = _ns.k_rule(rho, A64.shape[1])
        q = _ns.col_energy(A64)
        order = _ns._order(q) if hasattr(_ns, "_order") else np.argsort(-q, kind="stable")
        return np.sort(order[:k]), q

    def matmul(A, B, rho, _ns=ns):
        A64 = np.asarray(A, dtype=np.float64)
        B64 = np.asarray(B, dtype=np.float64)
        idx, _ = _ns.select(A64, rho)
        return idx, _ns._product(A64, B64, idx)

    def qk(Q, K, rho, heads=None, causal=False, _ns=ns):
        Q64 = np.asarray(Q, dtype=np.float64)
        K64 = np.asarray(K, dtype=np.float64)
        hq, tq, dh = Q64.shape
        hkv, tk, _ = K64.shape
        if causal and tq > tk:
            raise ValueError("tq > tk")
        out_i, out_s = [], []
        for h in range(hq):
            g = _ns.kv_head(h, hq, hkv)
            I, _ = _ns.select(Q64[h], rho)
            out_i.append(I)
            Sh = Q64[h][:, I] @ K64[g][:, I].T
            if causal:
                for row in range(tq):
                    for t in range(tk):
                        if not _ns._visible(row, t, tq, tk):
                            Sh[row, t] = _ns._masked
            out_s.append(Sh)
        return np.array(out_i), np.array(out_s)

    def pv(P, V, rho, _ns=ns):
        P64 = np.asarray(P, dtype=np.float64)
        V64 = np.asarray(V, dtype=np.float64)
        h_, tq, tk = P64.shape
        hkv = V64.shape[0]
        out_i, out_o = [], []
        for h in range(h_):
            g = _ns.kv_head(h, h_, hkv)
            I, _ = _ns.select(P64[h], rho)
            out_i.append(I)
            out_o.append(P64[h][:, I] @ V64[g][I, :])
        return np.array(out_i), np.array(out_o)

    if not hasattr(ns, "_visible"):
        ns._visible = lambda row, t, tq, tk: t <= row + tk - tq
    if not hasattr(ns, "_masked"):
        ns._masked = -np.inf
    if not hasattr(ns, "_product"):
        ns._product = lambda A, B, idx: A[:, idx] @ B[idx, :]
    if "select" not in over:
        ns.select = select
    ns.matmul = matmul
    ns.qk = qk
    ns.pv = pv
    return ns


MUTANTS = {
    "row_norms_instead_of_column": dict(col_energy=lambda A: np.sum(np.asarray(A, float) ** 2, axis=1)
                                        if np.asarray(A).shape[0] == np.asarray(A).shape[1]
                                        else np.resize(np.sum(np.asarray(A, float) ** 2, axis=1), np.asarray(A).shape[1])),
    "l1_instead_of_l2": dict(col_energy=lambda A: np.sum(np.abs(np.asarray(A, float)), axis=0)),
    "smallest_instead_of_largest": dict(_order=lambda q: np.argsort(q, kind="stable")),
    "highest_index_wins_ties": dict(_order=lambda q: (len(q) - 1 - np.argsort(-q[::-1], kind="stable"))),
    "floor_instead_of_ceil": dict(k_rule=lambda rho, d: max(1, int(math.floor(rho * d)))),
    "bare_binary_ceil": dict(k_rule=lambda rho, d: min(d, max(1, int(math.ceil(rho * d))))),
    "drops_kept_rows_of_B": dict(_product=lambda A, B, idx: A[:, idx] @ B[np.sort(np.setdiff1d(np.arange(B.shape[0]), idx))[:len(idx)], :]
                                 if len(idx) < B.shape[0] else A @ B),
    "w8_scale_per_row": dict(matmul_w8=lambda A, Bq, s, rho: (lambda I: (I, np.asarray(A, float)[:, I] @ (
        np.asarray(Bq, float)[I, :] * np.resize(np.asarray(s, float), len(I))[:, None])))(O.select(A, rho)[0])),
    "w8_read_unsigned": dict(matmul_w8=lambda A, Bq, s, rho: O.matmul_w8(A, np.asarray(Bq).view(np.uint8), s, rho)),
    "w8_scale_dropped": dict(matmul_w8=lambda A, Bq, s, rho: O.matmul_w8(A, Bq, np.ones_like(np.asarray(s, float)),
                                                                         rho)),
    "causal_top_left_aligned": dict(_visible=lambda row, t, tq, tk: t <= row),
    "causal_hides_the_diagonal": dict(_visible=lambda row, t, tq, tk: t < row + tk - tq),
    "causal_masks_with_zero": dict(_masked=0.0),
    "gqa_modulo_mapping": dict(kv_head=lambda h, hq, hkv: h % hkv),
    "product_sign_flip": dict(_product=lambda A, B, idx: -(A[:, idx] @ B[idx, :])),
    "dense_instead_of_reduced": dict(_product=lambda A, B, idx: A @ B),
    "dense_drops_last_term": dict(dense=lambda A, B: np.asarray(A, float)[:, :-1] @ np.asarray(B, float)[:-1, :]),
    "dense_in_float32": dict(dense=lambda A, B: (np.asarray(A, np.float32) @ np.asarray(B, np.float32)).astype(float)),
    "given_list_repeats_counted_once": dict(matmul_given=lambda A, B, idx: np.asarray(A, float)[:, np.unique(
        [t for t in np.asarray(idx) if 0 <= t < np.asarray(A).shape[1]]).astype(int)] @ np.asarray(B, float)[np.unique(
        [t for t in np.asarray(idx) if 0 <= t < np.asarray(A).shape[1]]).astype(int), :]),
    "softmax_without_max_shift_and_sign": dict(softmax_rows=lambda L, scale=1.0: np.exp(-np.asarray(L, float)) / np.sum(
        np.exp(-np.asarray(L, float)), axis=-1, keepdims=True)),
    "softmax_ignores_scale": dict(softmax_rows=lambda L, scale=1.0: O.softmax_rows(L)),
    "pv_energy_smallest_kept": dict(pv_given_energy=lambda P, V, E, rho, heads=None: O.pv_given_energy(P, V, -np.asarray(E), rho, heads)),
    "retained_over_dropped": dict(retained_energy=lambda A, rho: (lambda i_q: float(np.sum(i_q[1]) - np.sum(i_q[1][i_q[0]]))
                                   / max(float(np.sum(i_q[1])), 1e-300))(O.select(A, rho))),
    "given_list_negative_wraps": dict(matmul_given=lambda A, B, idx: np.asarray(A, float)[:, [t for t in np.asarray(idx)
        if t < np.asarray(A).shape[1]]] @ np.asarray(B, float)[[t for t in np.asarray(idx) if t < np.asarray(A).shape[1]], :]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # some planted mistakes overflow on purpose
def test_planted_mistake_fails_a_pin(name):
    ns = _mutant(**MUTANTS[name])
    failures = []
    for pin in PINS:
        try:
            msg = pin(ns)
        except Exception as e:  # a crash also counts as caught
            msg = f"raised {type(e).__name__}"
        if msg is not None:
            failures.append(pin.__name__)
    assert failures, f"mutant {name} passed every pin"


def test_unmutated_rebuild_passes_every_pin():
    ns = _mutant()
    for pin in PINS:
        assert pin(ns) is None, pin.__name__
