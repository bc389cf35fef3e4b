"""Seeded synthetic inputs for the RMM workloads.

Shared by the tests (both the oracle side and the HIP side read the same
stored tensors) and by the benchmark.  This module holds none of the method:
it never selects an index set, never forms a product and never returns a
score.  Its one look at the data is the column energy of its own draft,
used only to widen the score gap at each selection boundary so that the
kept set is well defined at float32 precision (acceptance needs neighbouring
sorted scores to differ by more than 1e-3 relative).

Recipes (shapes of the Llama-3.1 8B / 70B products the pages time; the
pages publish no inputs, so every value here is synthetic):

* activations A: z * c_j, z ~ N(0, 1), per-channel scale c_j = exp(N(0, 1))
  (log-normal, sigma = 1); the MLP workloads also scale round(1% of d)
  random "outlier" channels by 20.
* weights B: N(0, std) with std = 1 / sqrt(d) unless stated.
* attention: Q, K Gaussian with a per-(head, feature) log-normal scale;
  P = row softmax of N(0, std 2) logits; V ~ N(0, 1).
* bf16 tensors are rounded from float32 with round-to-nearest-even.

"N(0, x)" is read as mean 0 and standard deviation x.

Seeds: numpy PCG64 seeded from (1000 + workload number, part).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

GAP_REQUIRED = 1e-3   # acceptance: neighbouring sorted scores differ by more
GAP_TARGET = 1.5e-3   # what the generator aims for at each boundary
# With strict_adjacent every neighbouring pair of sorted scores is separated
# (the literal reading of the acceptance rule), which needs a spread of
# about (1 + gap)^d between the largest and smallest norm: for wide rows the
# generator aims just above the required gap so the spread stays moderate
# (1.00125^14336 is about 6e7 in norm, 4e15 in energy, far below fp32 range).
GAP_STRICT = 1.25e-3


def rng(workload: int, part: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + workload, part])))


def ceil_keep(rho: float, d: int) -> int:
    """Boundary position for a retention ratio (for spacing the draft only).

    Mirrors the documented k rule (decimal reading of rho * d) so the
    generator knows where to widen gaps; the product code and the oracle each
    compute k on their own.
    """
    x = rho * d
    r = round(x)
    k = int(r) if abs(x - r) <= 1e-9 * max(1.0, x) else int(math.ceil(x))
    return min(max(k, 1), d)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def to_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


def stored64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a stored (bf16 or fp32) CPU tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _draft_col_norms(t: torch.Tensor) -> np.ndarray:
    """Column L2 norms of a stored 2-D draft, float64, row-chunked."""
    x = t.detach().to("cpu")
    n = x.shape[0]
    acc = np.zeros(x.shape[1], dtype=np.float64)
    step = max(1, (1 << 22) // max(1, x.shape[1]))
    for r0 in range(0, n, step):
        blk = x[r0:r0 + step].to(torch.float64).numpy()
        acc += np.einsum("ij,ij->j", blk, blk)
    return np.sqrt(acc)


def _gaps(s: np.ndarray, ks) -> dict:
    order = np.argsort(-s, kind="stable")
    d = s.shape[0]
    out = {}
    for k in ks:
        if 0 < k < d:
            a, b = s[order[k - 1]], s[order[k]]
            out[int(k)] = float((a - b) / a) if a > 0 else 0.0
    return out


def _space_columns(z: np.ndarray, mult: np.ndarray, store, ks, literal: bool,
                   tries: int = 12, target: float = GAP_TARGET):
    """Rescale columns of draft z * mult until the required gaps hold.

    ks: boundary positions (k values) whose gap must exceed `target`.
    literal: every neighbouring pair must exceed it (cumulative stretch).
    store: maps a float32 draft to the stored tensor (bf16 or fp32).
    Returns (stored tensor, min gap at the checked positions).
    """
    mult = mult.astype(np.float64).copy()
    d = z.shape[1]
    check = list(range(1, d)) if literal else list(ks)
    factor = 1.0 + 2 * target
    for _ in range(tries):
        t = store((z * mult.astype(np.float32)[None, :]).astype(np.float32))
        s = _draft_col_norms(t)
        gaps = _gaps(s, check)
        worst = min(gaps.values()) if gaps else 1.0
        if worst > target:
            return t, worst
        order = np.argsort(-s, kind="stable")
        if literal:
            # walk from the smallest score up; each must exceed the one below
            # it by the factor
            up = order[::-1]
            t_prev = None
            for j in up:
                tj = s[j] if t_prev is None else max(s[j], t_prev * factor)
                if s[j] > 0:
                    mult[j] *= tj / s[j]
                t_prev = tj
        else:
            for k, g in sorted(gaps.items(), reverse=True):
                if g <= target:
                    mult[order[k:]] /= factor
        factor = 1.0 + (factor - 1.0) * 1.5
    raise RuntimeError("could not space the selection boundaries")


def _spacing(ks, strict: bool, d: int):
    """(boundaries, literal, target) for _space_columns: the selection
    boundaries of the workload, or every neighbouring pair when strict."""
    if strict:
        return (), True, (GAP_STRICT if d > 256 else GAP_TARGET)
    return ks, False, GAP_TARGET


@dataclass
class Workload:
    name: str
    tensors: dict
    rhos: tuple
    meta: dict = field(default_factory=dict)


def _activation(g: np.random.Generator, n: int, d: int, outlier_frac: float):
    z = g.standard_normal((n, d), dtype=np.float32)
    c = np.exp(g.standard_normal(d))
    if outlier_frac > 0:
        n_out = int(round(outlier_frac * d))
        out = g.choice(d, size=n_out, replace=False)
        c[out] *= 20.0
    return z, c


def tiny_projection(n=16, d=256, m=256, rho=0.5, strict_adjacent=True) -> Workload:
    """A n x d fp32, literal score separation; B d x m fp32 N(0, 1/sqrt(d))."""
    g = rng(0)
    z = g.standard_normal((n, d), dtype=np.float32)
    c = np.exp(g.standard_normal(d))
    # make the scales strictly distinct (they already are with probability 1)
    A, gap = _space_columns(z, c, to_f32, (), literal=True)
    B = to_f32(g.standard_normal((d, m), dtype=np.float32) / np.float32(math.sqrt(d)))
    return Workload("tiny_projection_fp32", {"A": A, "B": B}, (rho,),
                    {"n": n, "d": d, "m": m, "dtype": "fp32", "min_gap": gap})


def mlp_down(n=4096, d=14336, m=4096, rhos=(0.9, 0.7, 0.5), workload=1, strict_adjacent=False) -> Workload:
    """Llama-3.1-8B MLP down projection, prefill: A n x d, B d x m, bf16."""
    g = rng(workload)
    z, c = _activation(g, n, d, 0.01)
    ks = sorted({ceil_keep(r, d) for r in rhos if r < 1.0}, reverse=True)
    ks, literal, target = _spacing(ks, strict_adjacent, d)
    A, gap = _space_columns(z, c, to_bf16, ks, literal=literal, target=target)
    del z
    B = to_bf16(g.standard_normal((d, m), dtype=np.float32) / np.float32(math.sqrt(d)))
    return Workload("mlp_down_8b", {"A": A, "B": B}, tuple(rhos),
                    {"n": n, "d": d, "m": m, "dtype": "bf16", "min_gap": gap, "strict_adjacent": strict_adjacent})


def mlp_up(n=2048, d=8192, m=28672, rho=0.8, strict_adjacent=False) -> Workload:
    """Llama-3.1-70B MLP up projection: A n x d (MLP-down recipe), B d x m."""
    w = mlp_down(n=n, d=d, m=m, rhos=(rho,), workload=4, strict_adjacent=strict_adjacent)
    w.name = "mlp_up_70b"
    return w


def decode_qkv(n=8, d=4096, m=6144, rho=0.8, strict_adjacent=False) -> Workload:
    """Decode-shaped fused QKV projection: A n x d, B d x m (std 1/sqrt(d))."""
    g = rng(3)
    z, c = _activation(g, n, d, 0.0)
    ks, literal, target = _spacing((ceil_keep(rho, d),), strict_adjacent, d)
    A, gap = _space_columns(z, c, to_bf16, ks, literal=literal, target=target)
    B = to_bf16(g.standard_normal((d, m), dtype=np.float32) / np.float32(math.sqrt(d)))
    return Workload("decode_qkv_8b", {"A": A, "B": B}, (rho,),
                    {"n": n, "d": d, "m": m, "dtype": "bf16", "min_gap": gap, "strict_adjacent": strict_adjacent})


def int8_weights(g: np.random.Generator, d: int, m: int):
    """Weights N(0, 1/sqrt(d)) stored as symmetric per-output-column int8:
    scale[c] = max_j |B[j, c]| / 127 and Bq = round(B / scale) in [-127, 127].
    Returns (Bq int8 tensor, scale fp32 tensor)."""
    Bq = np.empty((d, m), dtype=np.int8)
    scale = np.empty(m, dtype=np.float32)
    step = max(1, (1 << 24) // max(1, d))
    for c0 in range(0, m, step):
        blk = g.standard_normal((d, min(step, m - c0)), dtype=np.float32) / np.float32(math.sqrt(d))
        sc = np.maximum(np.max(np.abs(blk), axis=0), np.float32(1e-30)) / np.float32(127.0)
        Bq[:, c0:c0 + blk.shape[1]] = np.clip(np.rint(blk / sc), -127, 127).astype(np.int8)
        scale[c0:c0 + blk.shape[1]] = sc
    return torch.from_numpy(Bq), torch.from_numpy(scale)


def w8_projection(n=8, d=4096, m=6144, rho=0.8, workload=5, name="decode_qkv_8b_w8",
                  strict_adjacent=False) -> Workload:
    """A n x d bf16 (MLP-down activation recipe, boundary separation at rho)
    with int8 weights of d x m (int8_weights)."""
    g = rng(workload)
    z, c = _activation(g, n, d, 0.01 if n > 64 else 0.0)
    ks, literal, target = _spacing((ceil_keep(rho, d),) if rho < 1.0 else (), strict_adjacent, d)
    A, gap = _space_columns(z, c, to_bf16, ks, literal=literal, target=target)
    del z
    Bq, scale = int8_weights(g, d, m)
    return Workload(name, {"A": A, "Bq": Bq, "scale": scale}, (rho,),
                    {"n": n, "d": d, "m": m, "dtype": "bf16 x int8", "min_gap": gap})


def gqa_qk(hq=32, hkv=8, t=4096, dh=128, rho=0.5, strict_adjacent=True) -> Workload:
    """QK^T prefill: Q (hq, t, dh), K (hkv, t, dh) bf16, per-feature scales.

    Every query head gets literal separation of its dh column norms.
    """
    g = rng(2)
    Qs = []
    gaps = []
    for h in range(hq):
        z = g.standard_normal((t, dh), dtype=np.float32)
        c = np.exp(g.standard_normal(dh))
        q, gap = _space_columns(z, c, to_bf16, (), literal=True)
        Qs.append(q)
        gaps.append(gap)
    Q = torch.stack(Qs, 0)
    zk = g.standard_normal((hkv, t, dh), dtype=np.float32)
    ck = np.exp(g.standard_normal((hkv, 1, dh))).astype(np.float32)
    K = to_bf16(zk * ck)
    return Workload("gqa_qk_8b", {"Q": Q, "K": K}, (rho,),
                    {"hq": hq, "hkv": hkv, "t": t, "dh": dh, "dtype": "bf16",
                     "min_gap": float(min(gaps))})


def decode_attn_qk(hq=32, hkv=8, tq=1, tk=8192, dh=128, rho=0.5, strict_adjacent=True) -> Workload:
    """Decode QK^T: Q (hq, tq, dh) with literal separation of each head's
    feature norms over its tq rows; a key cache K (hkv, tk, dh); bf16."""
    g = rng(6)
    Qs = []
    gaps = []
    for _ in range(hq):
        z = g.standard_normal((tq, dh), dtype=np.float32)
        c = np.exp(g.standard_normal(dh))
        q, gap = _space_columns(z, c, to_bf16, (), literal=True)
        Qs.append(q)
        gaps.append(gap)
    Q = torch.stack(Qs, 0)
    zk = g.standard_normal((hkv, tk, dh), dtype=np.float32)
    ck = np.exp(g.standard_normal((hkv, 1, dh))).astype(np.float32)
    K = to_bf16(zk * ck)
    return Workload("decode_attn_qk", {"Q": Q, "K": K}, (rho,),
                    {"hq": hq, "hkv": hkv, "tq": tq, "tk": tk, "dh": dh, "min_gap": float(min(gaps))})


def _softmax_rows(L: np.ndarray) -> np.ndarray:
    m = L.max(axis=1, keepdims=True)
    e = np.exp(L - m)
    return e / e.sum(axis=1, keepdims=True)


def attn_pv(h=64, hkv=8, tq=512, tk=8192, dv=128, rho=0.5, with_logits=False, strict_adjacent=False) -> Workload:
    """PV: P (h, tq, tk) fp32 = row softmax of N(0, std 2) logits; V (hkv, tk, dv).

    The boundary gap of each head is widened by lowering the logits of the
    key positions ranked below the boundary (rows stay stochastic).  With
    `strict_adjacent` every neighbouring pair of sorted key norms is spaced
    instead (cumulative logit shifts, walked from the smallest norm up).
    With `with_logits` the shifted logits L (fp32) whose softmax P is are
    kept too.
    """
    g = rng(4, part=1)
    k = ceil_keep(rho, tk)
    P = torch.empty((h, tq, tk), dtype=torch.float32)
    Ls = torch.empty((h, tq, tk), dtype=torch.float32) if with_logits else None
    gaps = []
    check = list(range(1, tk)) if strict_adjacent else [k]
    target = (GAP_STRICT if tk > 256 else GAP_TARGET) if strict_adjacent else GAP_TARGET
    for hh in range(h):
        L = 2.0 * g.standard_normal((tq, tk))
        shift = np.zeros(tk)
        step = math.log(1.0 + 2 * target)
        for _ in range(16):
            Ph = to_f32(_softmax_rows(L + shift[None, :]))
            s = _draft_col_norms(Ph)
            gp = _gaps(s, check)
            gap = min(gp.values()) if gp else 1.0
            if gap > target:
                break
            order = np.argsort(-s, kind="stable")
            if strict_adjacent:
                # each norm, walking up from the smallest, must exceed the one
                # below it by the step: raise its logit by the missing factor
                t_prev = None
                for j in order[::-1]:
                    tj = s[j] if t_prev is None else max(s[j], t_prev * math.exp(step))
                    if s[j] > 0:
                        shift[j] += math.log(tj / s[j])
                    t_prev = tj
            else:
                shift[order[k:]] -= step
            step *= 1.5
        else:
            raise RuntimeError("could not space the PV key norms")
        P[hh] = Ph
        if with_logits:
            Ls[hh] = to_f32(L + shift[None, :])
        gaps.append(gap)
    V = to_bf16(g.standard_normal((hkv, tk, dv), dtype=np.float32))
    tensors = {"P": P, "V": V}
    if with_logits:
        tensors["L"] = Ls
    return Workload("attn_pv_70b", tensors, (rho,),
                    {"h": h, "hkv": hkv, "tq": tq, "tk": tk, "dv": dv,
                     "dtype": "fp32/bf16", "min_gap": float(min(gaps)), "strict_adjacent": strict_adjacent})


# The workloads named by the benchmark configuration list, in its order.
FULL = {
    "tiny_projection": tiny_projection,
    "mlp_down_8b": mlp_down,
    "gqa_qk_8b": gqa_qk,
    "decode_qkv_8b": decode_qkv,
    "mlp_up_70b": mlp_up,
    "attn_pv_70b": attn_pv,
}
