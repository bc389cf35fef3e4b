"""Plain CPU oracle for Reduced Matrix Multiplication (RMM).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the tests, the smoke check of the build entry point
and the benchmark's CPU-baseline leg use it.  It shares no code, header,
table or helper with the HIP library.

What it computes (everything in float64, from the exact stored input bits;
bf16 and fp32 values convert to float64 without rounding):

* k rule      -- |I| = ceil(rho * d) for rho in (0, 1].
                 Source: hackcv.com "Algorithm Deep-Dive: RMM", section
                 "Core Approach (Formula Level) / Contraction-Dimension TopK
                 Selection"; gist.science "Reduced Matrix Multiplication",
                 Technical Summary, "Selection Strategy".
* scores      -- s_j = ||A[:, j]||_2, the L2 norm of column j of the
                 activation matrix A (n x d) over all n rows.  Ranking uses
                 q_j = s_j**2, which orders the columns identically.
                 Source: hackcv.com, same section ("importance score");
                 kaelemshawn.blog, section on why fewer multiply-adds can
                 suffice (the column L2 norm as importance).
* selection   -- the k indices with the largest scores; among equal scores
                 the lower index wins; the set is returned in ascending order.
                 The pages only say the selection is deterministic for a
                 given input; lowest-index tie-breaking and ascending output
                 are the readings this oracle fixes.
* product     -- Y = A[:, I] @ B[I, :]  (hackcv.com, "Core Approach":
                 RMM_rho(A, B)).  Only the kept rows of B take part.
* QK^T        -- per query head h: I_h from the column norms of Q[h]
                 (tokens x head_dim) over its query rows, and
                 S_h = Q[h][:, I_h] @ K[g(h)][:, I_h]^T, where K/V head
                 g(h) = h // (hq // hkv) serves query head h (grouped-query
                 attention: selection on Q, K gathers the same feature
                 dims).  Source: hackcv.com "Component mapping"; kaelemshawn
                 .blog section on where RMM cuts inside the Transformer.
* retained    -- sum of the kept energies over the sum of all energies.
* producer    -- P = row softmax of logits (float64) and, per head, the
                 column energies of P: the PV scores emitted by the pass
                 that writes P; pv_given_energy selects on supplied scores.
* given I     -- Y = sum over the entries t of a caller-given list of
                 A[:, t] B[t, :] (entries outside [0, d) ignored).
* int8 B      -- Y = A[:, I] @ (Bq[I, :] * s[None, :]): weights stored as
                 int8 with one scale per output column (symmetric per-channel
                 quantisation; the pages say RMM combines with INT8 weight
                 quantisation but give no scheme, so this plainest reading
                 is the one fixed here).  Selection is unchanged: it reads A.
                 Source: hackcv.com, "Compatibility & generalization";
                 gist.science, Experimental Results (the compatibility item).
* PV          -- per head h: I_h from the column norms of P[h]
                 (queries x keys) over its query rows (the token axis is the
                 contraction axis), and O_h = P[h][:, I_h] @ V[g(h)][I_h, :].
                 Same sources.

No blocking, fusion or reordering beyond these definitions.  A library
matmul serves as the product step; a stable argsort serves as the ranking
step.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "k_rule",
    "col_energy",
    "select",
    "matmul",
    "matmul_given",
    "matmul_w8",
    "dense",
    "qk",
    "pv",
    "softmax_rows",
    "pv_given_energy",
    "kv_head",
    "error_bound",
    "retained_energy",
]


def k_rule(rho: float, d: int) -> int:
    """Number of kept contraction indices, ceil(rho * d).

    hackcv.com "Algorithm Deep-Dive: RMM", Core Approach: |I| = ceil(rho d);
    the retention-ratio knob section: rho lies in (0, 1].

    Reading (the pages are silent on floating-point rounding of rho * d):
    rho is the decimal the caller wrote, so a product that lands within
    1e-9 relative of an integer is that integer.  Example: 0.07 * 100 is
    7.000000000000001 in binary floating point; a bare ceil would keep 8
    columns where the caller asked for 7.
    """
    if isinstance(rho, bool) or not isinstance(rho, (int, float, np.floating)):
        raise TypeError("rho must be a real number")
    rho = float(rho)
    if not math.isfinite(rho) or rho <= 0.0 or rho > 1.0:
        raise ValueError(f"rho must lie in (0, 1], got {rho!r}")
    d = int(d)
    if d < 1:
        raise ValueError(f"d must be >= 1, got {d}")
    x = rho * d
    r = round(x)
    if abs(x - r) <= 1e-9 * max(1.0, x):
        k = int(r)
    else:
        k = int(math.ceil(x))
    return min(max(k, 1), d)


def col_energy(A) -> np.ndarray:
    """q_j = sum_i A[i, j]**2 in float64 (the squared column L2 norm)."""
    A64 = np.asarray(A, dtype=np.float64)
    if A64.ndim != 2:
        raise ValueError("A must be 2-D (rows x contraction)")
    return np.sum(A64 * A64, axis=0)


def select(A, rho: float):
    """Indices of the ceil(rho d) largest column norms of A, ascending.

    Ranking key: descending q_j; equal keys keep ascending index order
    (stable sort), so the lowest index wins a tie.  Returns (idx, q) with
    idx int64 of length k, sorted ascending, and q the float64 energies.
    """
    A64 = np.asarray(A, dtype=np.float64)
    d = A64.shape[1]
    k = k_rule(rho, d)
    q = col_energy(A64)
    order = np.argsort(-q, kind="stable")
    idx = np.sort(order[:k])
    return idx.astype(np.int64), q


def matmul(A, B, rho: float, rows=None):
    """RMM_rho(A, B) = A[:, I] @ B[I, :] with I = select(A, rho).

    A: n x d, B: d x m.  Returns (idx, Y) with Y float64 n x m.  With
    `rows`, Y holds only those rows of the product; the selection still
    uses every row of A.
    """
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    if A64.ndim != 2 or B64.ndim != 2 or A64.shape[1] != B64.shape[0]:
        raise ValueError("need A (n x d) and B (d x m)")
    idx, _ = select(A64, rho)
    Ar = A64 if rows is None else A64[np.asarray(rows)]
    Y = Ar[:, idx] @ B64[idx, :]
    return idx, Y


def matmul_given(A, B, idx) -> np.ndarray:
    """The reduced product over an index list the caller supplies:
    Y = sum over the entries t of idx of A[:, t] B[t, :].

    This is RMM_rho(A, B) = A[:, I] B[I, :] (hackcv.com, "Core Approach")
    with I given instead of selected, as when one selection on X serves
    several projections or a random set of the same size replaces it
    (gist.science, Selection Strategy, random-selection comparison).  The
    list may be in any order; a repeated entry counts once per occurrence;
    an entry outside [0, d) contributes nothing (the reading the library's
    interface fixes for invalid entries).  Returns float64 n x m.
    """
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    d = A64.shape[1]
    I = np.asarray(idx, dtype=np.int64).ravel()
    I = I[(I >= 0) & (I < d)]
    return A64[:, I] @ B64[I, :]


def matmul_w8(A, Bq, scale, rho: float, rows=None):
    """Reduced product with int8 weights and a float scale per output column.

    The weights are B[j, c] = Bq[j, c] * scale[c] (symmetric per-output-
    channel int8, the reading of "INT8 weight quantisation" fixed here), so
    Y = A[:, I] @ (Bq[I, :] * scale) with I the TopK of A's column norms,
    exactly as for float weights.  Bq holds integers in [-128, 127].
    Returns (idx, Y) with Y float64 n x m (only `rows` of it if given; the
    selection still uses every row of A).
    """
    A64 = np.asarray(A, dtype=np.float64)
    s64 = np.asarray(scale, dtype=np.float64).ravel()
    if np.asarray(Bq).shape[1] != s64.shape[0]:
        raise ValueError("one scale per column of Bq")
    idx, _ = select(A64, rho)
    Ar = A64 if rows is None else A64[np.asarray(rows)]
    Bk = np.asarray(Bq)[idx, :].astype(np.float64)
    return idx, Ar[:, idx] @ (Bk * s64[None, :])


def dense(A, B) -> np.ndarray:
    """The unreduced product A @ B in float64."""
    return np.asarray(A, dtype=np.float64) @ np.asarray(B, dtype=np.float64)


def kv_head(h: int, hq: int, hkv: int) -> int:
    """K/V head serving query head h under grouped-query attention.

    The pages say selection happens on Q per head and K/V gather the
    matching dims; which K/V head pairs with which Q head is not stated.
    Reading: contiguous groups of hq // hkv query heads share one K/V head
    (the Llama convention).
    """
    if hq % hkv != 0:
        raise ValueError("hq must be a multiple of hkv")
    return h // (hq // hkv)


def qk(Q, K, rho: float, heads=None, causal: bool = False):
    """Per-head reduced attention scores.

    Q: (hq, tq, dh), K: (hkv, tk, dh).  For each query head h, I_h is chosen
    from the column norms of Q[h] (over its tq rows) and
    S[h] = Q[h][:, I_h] @ K[g(h)][:, I_h]^T.  Raw product: no 1/sqrt(dh)
    scale (the softmax takes it).  With `causal`, the tq queries are the last
    tq positions of the tk keys (tq <= tk), so query row r sees keys
    t <= r + tk - tq and every later key gets -inf; the mask acts on the
    scores only, the selection still reads every row of Q[h].
    Returns (idx (hq, k) int64, S (hq, tq, tk) float64).  With `heads`,
    idx and S cover only those query heads, in the order given.
    """
    Q = np.asarray(Q)
    K = np.asarray(K)
    hq, tq, dh = Q.shape
    hkv, tk, dh2 = K.shape
    if dh2 != dh:
        raise ValueError("Q and K head dims differ")
    if causal and tq > tk:
        raise ValueError("causal scores need tq <= tk")
    hs = list(range(hq)) if heads is None else [int(h) for h in heads]
    k = k_rule(rho, dh)
    idx = np.empty((len(hs), k), dtype=np.int64)
    S = np.empty((len(hs), tq, tk), dtype=np.float64)
    for i, h in enumerate(hs):
        g = kv_head(h, hq, hkv)
        Qh = np.asarray(Q[h], dtype=np.float64)
        Kg = np.asarray(K[g], dtype=np.float64)
        I, _ = select(Qh, rho)
        idx[i] = I
        S[i] = Qh[:, I] @ Kg[:, I].T
        if causal:
            for r in range(tq):
                S[i, r, r + tk - tq + 1:] = -np.inf
    return idx, S


def pv(P, V, rho: float, heads=None):
    """Per-head reduced attention output over the key (token) axis.

    P: (h, tq, tk) attention weights, V: (hkv, tk, dv).  For each head h,
    I_h is chosen from the column norms of P[h] over its tq query rows and
    O[h] = P[h][:, I_h] @ V[g(h)][I_h, :].
    Returns (idx (h, k) int64, O (h, tq, dv) float64).  With `heads`, idx
    and O cover only those heads, in the order given.
    """
    P = np.asarray(P)
    V = np.asarray(V)
    h_, tq, tk = P.shape
    hkv, tk2, dv = V.shape
    if tk2 != tk:
        raise ValueError("P key axis and V rows differ")
    hs = list(range(h_)) if heads is None else [int(h) for h in heads]
    k = k_rule(rho, tk)
    idx = np.empty((len(hs), k), dtype=np.int64)
    O = np.empty((len(hs), tq, dv), dtype=np.float64)
    for i, h in enumerate(hs):
        g = kv_head(h, h_, hkv)
        Ph = np.asarray(P[h], dtype=np.float64)
        Vg = np.asarray(V[g], dtype=np.float64)
        I, _ = select(Ph, rho)
        idx[i] = I
        O[i] = Ph[:, I] @ Vg[I, :]
    return idx, O


def error_bound(A, B, idx) -> float:
    """Right-hand side of the pages' Frobenius error bound.

    hackcv.com "Algorithm Deep-Dive: RMM", Core Approach, Properties:
    ||AB - A[:, I] B[I, :]||_F <= sum over dropped j of
    ||A[:, j]||_2 * ||B[j, :]||_2.
    """
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    keep = np.zeros(A64.shape[1], dtype=bool)
    keep[np.asarray(idx)] = True
    drop = ~keep
    s = np.sqrt(col_energy(A64))
    b = np.sqrt(np.sum(B64 * B64, axis=1))
    return float(np.sum(s[drop] * b[drop]))


def softmax_rows(L, scale: float = 1.0) -> np.ndarray:
    """Row softmax in float64 over the last axis of x = scale * L:
    exp(x - max x) / sum exp(x - max x) (scale = 1/sqrt(head dim) for raw
    QK^T scores).

    P, the attention weights that the PV product contracts over key
    positions (kaelemshawn.blog, section on where RMM cuts inside the
    Transformer), is this softmax of the logits row by row; the pass that
    writes it can also emit col_energy(P) per head, the PV scores.
    """
    L64 = float(scale) * np.asarray(L, dtype=np.float64)
    m = np.max(L64, axis=-1, keepdims=True)
    e = np.exp(L64 - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def pv_given_energy(P, V, energy, rho: float, heads=None):
    """PV with the key scores supplied: for each head h, I_h holds the
    ceil(rho tk) key positions of largest energy[h] (ties to the lower
    index, ascending) and O_h = P[h][:, I_h] @ V[g(h)][I_h, :].  With
    energy = column energies of P this is pv(P, V, rho).  Returns
    (idx (h, k) int64, O (h, tq, dv) float64); `heads` as in pv.
    """
    P = np.asarray(P)
    V = np.asarray(V)
    E = np.asarray(energy, dtype=np.float64)
    h_, tq, tk = P.shape
    hkv, _, dv = V.shape
    hs = list(range(h_)) if heads is None else [int(h) for h in heads]
    k = k_rule(rho, tk)
    idx = np.empty((len(hs), k), dtype=np.int64)
    O = np.empty((len(hs), tq, dv), dtype=np.float64)
    for i, h in enumerate(hs):
        g = kv_head(h, h_, hkv)
        order = np.argsort(-E[h], kind="stable")
        I = np.sort(order[:k])
        idx[i] = I
        O[i] = np.asarray(P[h], dtype=np.float64)[:, I] @ np.asarray(V[g], dtype=np.float64)[I, :]
    return idx, O


def retained_energy(A, rho: float) -> float:
    """Fraction of the activation energy the selection keeps:
    sum over kept j of q_j / sum over all j of q_j (1.0 when every column is
    kept).  hackcv.com, "Attention vs MLP: structural asymmetry" (the
    supplementary figures quote it per reduced component); kaelemshawn.blog,
    the compute-normalized component analysis.
    """
    idx, q = select(A, rho)
    tot = float(np.sum(q))
    return 1.0 if tot == 0.0 else float(np.sum(q[idx])) / tot
