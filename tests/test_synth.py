"""The seeded generators: their k rule agrees with the oracle's, and the
score separation they promise holds on the stored values (CPU only)."""

import json
import math
import os
from fractions import Fraction

import numpy as np

import synth
from oracle import rmm_oracle as O
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_ceil_keep_matches_the_oracle_k_rule():
    # the generator widens gaps at the boundary the product will use: its
    # copy of the k rule must place that boundary where the oracle does
    with open(os.path.join(GOLDEN, "k_rule.json")) as f:
        for c in json.load(f)["cases"]:
            assert W.ceil_keep(c["rho"], c["d"]) == O.k_rule(c["rho"], c["d"]) == c["k"], c
    for num in range(1, 101):
        rho = float(f"{num / 100:.2f}")
        for d in (1, 3, 7, 10, 100, 128, 999, 4096, 8192, 14336):
            want = max(1, min(d, math.ceil(Fraction(f"{num / 100:.2f}") * d)))
            assert W.ceil_keep(rho, d) == O.k_rule(rho, d) == want, (rho, d)


def _sorted_gaps(q):
    s = np.sort(np.sqrt(np.asarray(q, dtype=np.float64)))[::-1]
    return (s[:-1] - s[1:]) / s[:-1]


def test_boundary_separation_default():
    w = synth.mlp_down(n=64, d=1500, m=8, rhos=(0.9, 0.7, 0.5))
    q = O.col_energy(synth.stored64(w.tensors["A"]))
    order = np.argsort(-q, kind="stable")
    s = np.sqrt(q)
    for rho in (0.9, 0.7, 0.5):
        k = O.k_rule(rho, 1500)
        a, b = s[order[k - 1]], s[order[k]]
        assert (a - b) / a > synth.GAP_REQUIRED, rho


def test_strict_adjacent_every_pair():
    # the literal reading: every neighbouring pair of sorted scores differs
    # by more than 1e-3 relative, on the stored bf16 / fp32 values
    w = synth.mlp_down(n=64, d=1500, m=8, rhos=(0.7,), strict_adjacent=True)
    assert _sorted_gaps(O.col_energy(synth.stored64(w.tensors["A"]))).min() > synth.GAP_REQUIRED
    w = synth.decode_qkv(n=8, d=1024, m=8, strict_adjacent=True)
    assert _sorted_gaps(O.col_energy(synth.stored64(w.tensors["A"]))).min() > synth.GAP_REQUIRED
    w = synth.w8_projection(n=8, d=700, m=16, strict_adjacent=True)
    assert _sorted_gaps(O.col_energy(synth.stored64(w.tensors["A"]))).min() > synth.GAP_REQUIRED
    w = synth.attn_pv(h=2, hkv=1, tq=16, tk=600, dv=8, strict_adjacent=True)
    P = synth.stored64(w.tensors["P"])
    for h in range(2):
        assert _sorted_gaps(O.col_energy(P[h])).min() > synth.GAP_REQUIRED
        assert np.allclose(P[h].sum(axis=1), 1.0, atol=1e-5)   # rows stay stochastic
