"""Thin Python binding of librmm (the C ABI in include/rmm.h).

Argument marshalling only: every step of RMM runs in the HIP library.
PyTorch provides device memory (inputs, outputs, workspace) and the current
stream.  The library must be built (python -m
input_adaptive_reduced_colnorm_amd.build); nothing here computes a fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librmm.so")

RMM_OK = 0
RMM_FP32 = 0
RMM_BF16 = 1

# operation codes of rmm_workspace_bytes (rmm_op_t)
OPS = {"select": 0, "matmul": 1, "qk": 2, "pv": 3, "matmul_w8": 4, "matmul_idx": 5, "softmax_energy": 6,
       "pv_energy": 7, "softmax_select": 8, "pv_idx": 9}

_c = ctypes
_vp, _i64, _dbl, _sz, _int = _c.c_void_p, _c.c_int64, _c.c_double, _c.c_size_t, _c.c_int

# name -> (restype, argtypes), mirroring include/rmm.h
SIGNATURES = {
    "rmm_k": (_i64, [_dbl, _i64]),
    "rmm_status_str": (_c.c_char_p, [_int]),
    "rmm_workspace_bytes": (_sz, [_int, _i64, _i64, _i64]),
    "rmm_select_workspace": (_sz, [_i64, _i64, _int]),
    "rmm_select": (_int, [_vp, _int, _i64, _i64, _i64, _dbl, _vp, _vp, _vp, _sz, _vp]),
    "rmm_select_retained": (_int, [_vp, _int, _i64, _i64, _i64, _dbl, _vp, _vp, _vp, _vp, _sz, _vp]),
    "rmm_matmul_workspace": (_sz, [_i64, _i64, _i64, _i64, _int, _dbl]),
    "rmm_matmul": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int, _i64, _vp, _sz, _vp]),
    "rmm_matmul_noalloc": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int, _i64, _vp]),
    "rmm_matmul_timed": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int, _i64, _vp, _sz,
                                _vp, _vp]),
    "rmm_matmul_w8_workspace": (_sz, [_i64, _i64, _i64, _i64, _dbl]),
    "rmm_matmul_w8": (_int, [_vp, _int, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int, _i64, _vp, _sz,
                             _vp]),
    "rmm_matmul_w8_timed": (_int, [_vp, _int, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int, _i64, _vp,
                                   _sz, _vp, _vp]),
    "rmm_matmul_idx_workspace": (_sz, [_i64, _i64, _i64, _int]),
    "rmm_matmul_idx": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _int, _i64, _vp, _sz,
                              _vp]),
    "rmm_qk_workspace": (_sz, [_i64, _i64, _i64, _i64, _int, _dbl]),
    "rmm_qk": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int,
                      _vp, _sz, _vp]),
    "rmm_qk_causal": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp, _int,
                      _vp, _sz, _vp]),
    "rmm_qk_timed": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp,
                            _int, _vp, _sz, _vp, _vp]),
    "rmm_pv_workspace": (_sz, [_i64, _i64, _i64, _i64, _int, _int, _dbl]),
    "rmm_pv": (_int, [_vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _dbl, _vp, _vp,
                      _int, _vp, _sz, _vp]),
    "rmm_softmax_energy_workspace": (_sz, [_i64, _i64, _i64]),
    "rmm_softmax_select_workspace": (_sz, [_i64, _i64, _i64]),
    "rmm_softmax_select": (_int, [_vp, _c.c_float, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _dbl, _vp,
                                  _vp, _sz, _vp]),
    "rmm_pv_idx_workspace": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "rmm_pv_idx": (_int, [_vp, _int, _vp, _int, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                          _vp, _int, _vp, _sz, _vp]),
    "rmm_softmax_energy": (_int, [_vp, _c.c_float, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _sz, _vp]),
    "rmm_pv_energy_workspace": (_sz, [_i64, _i64, _i64, _i64, _int, _int, _dbl]),
    "rmm_pv_energy": (_int, [_vp, _int, _vp, _int, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _dbl,
                             _vp, _vp, _int, _vp, _sz, _vp]),
    "rmm_pv_timed": (_int, [_vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _dbl, _vp,
                            _vp, _int, _vp, _sz, _vp, _vp]),
}

_lib = None


class RMMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def lib() -> ctypes.CDLL:
    """Loads librmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"librmm.so not built ({_LIB_PATH}); run python -m input_adaptive_reduced_colnorm_amd.build")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().rmm_status_str(int(status)).decode()


def k(rho: float, d: int) -> int:
    return int(lib().rmm_k(float(rho), int(d)))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RMM_FP32
    if t.dtype == torch.bfloat16:
        return RMM_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tdt(code: int):
    return torch.float32 if code == RMM_FP32 else torch.bfloat16


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check_dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must live on the same GPU")
    return dev


def _ws(nbytes: int, dev: torch.device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def _raise(st: int, where: str):
    if st != RMM_OK:
        raise RMMError(st, where)


def select(A: torch.Tensor, rho: float, scores: bool = False):
    """Kept index set of A (n x d, unit inner stride).  Returns idx or (idx, s)."""
    dev = _check_dev(A)
    n, d = A.shape
    if A.stride(1) != 1:
        raise ValueError("A needs unit inner stride")
    L = lib()
    kk = k(rho, d)
    idx = torch.empty(max(kk, 1), dtype=torch.int32, device=dev)
    sc = torch.empty(d, dtype=torch.float32, device=dev) if scores else None
    ws = _ws(L.rmm_select_workspace(n, d, _dt(A)), dev)
    st = L.rmm_select(A.data_ptr(), _dt(A), n, d, A.stride(0), float(rho), idx.data_ptr(),
                      sc.data_ptr() if sc is not None else None, ws.data_ptr(), ws.numel(), _stream(dev))
    _raise(st, "rmm_select")
    return (idx, sc) if scores else idx


def select_retained(A: torch.Tensor, rho: float):
    """Kept index set of A and the retained energy fraction (a 1-element fp32
    device tensor).  Returns (idx, retained)."""
    dev = _check_dev(A)
    n, d = A.shape
    if A.stride(1) != 1:
        raise ValueError("A needs unit inner stride")
    L = lib()
    kk = k(rho, d)
    idx = torch.empty(max(kk, 1), dtype=torch.int32, device=dev)
    ret = torch.empty(1, dtype=torch.float32, device=dev)
    ws = _ws(L.rmm_select_workspace(n, d, _dt(A)), dev)
    st = L.rmm_select_retained(A.data_ptr(), _dt(A), n, d, A.stride(0), float(rho), idx.data_ptr(), None,
                               ret.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _raise(st, "rmm_select_retained")
    return idx, ret


def matmul(A: torch.Tensor, B: torch.Tensor, rho: float, out_dtype=torch.float32, workspace: torch.Tensor = None,
           out: torch.Tensor = None, idx: torch.Tensor = None):
    """Y = A[:, I] B[I, :].  Returns (idx, Y)."""
    dev = _check_dev(A, B)
    n, d = A.shape
    d2, m = B.shape
    if d2 != d:
        raise ValueError("A and B disagree on the contraction size")
    if A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B need unit inner stride")
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    L = lib()
    kk = k(rho, d)
    if idx is None:
        idx = torch.empty(kk, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((n, m), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_matmul_workspace(n, d, m, A.stride(0), _dt(A), float(rho)), dev)
    st = L.rmm_matmul(A.data_ptr(), B.data_ptr(), _dt(A), n, d, m, A.stride(0), B.stride(0), float(rho),
                      idx.data_ptr(), out.data_ptr(), _dt(out), out.stride(0), workspace.data_ptr(),
                      workspace.numel(), _stream(dev))
    _raise(st, "rmm_matmul")
    return idx, out


def matmul_idx(A: torch.Tensor, B: torch.Tensor, idx: torch.Tensor, out_dtype=torch.float32,
               workspace: torch.Tensor = None, out: torch.Tensor = None) -> torch.Tensor:
    """Y = sum over t of A[:, idx[t]] B[idx[t], :] for a given int32 index list
    (entries outside [0, d) contribute nothing).  Returns Y."""
    dev = _check_dev(A, B)
    n, d = A.shape
    d2, m = B.shape
    if d2 != d:
        raise ValueError("A and B disagree on the contraction size")
    if A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B need unit inner stride")
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    if idx.dtype != torch.int32 or idx.dim() != 1 or not idx.is_contiguous() or idx.device != dev:
        raise TypeError("idx must be a contiguous 1-D int32 tensor on the same device")
    L = lib()
    kk = idx.numel()
    if out is None:
        out = torch.empty((n, m), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_matmul_idx_workspace(n, kk, m, _dt(A)), dev)
    st = L.rmm_matmul_idx(A.data_ptr(), B.data_ptr(), _dt(A), n, d, m, A.stride(0), B.stride(0), idx.data_ptr(), kk,
                          out.data_ptr(), _dt(out), out.stride(0), workspace.data_ptr(), workspace.numel(),
                          _stream(dev))
    _raise(st, "rmm_matmul_idx")
    return out


def matmul_w8(A: torch.Tensor, Bq: torch.Tensor, scale: torch.Tensor, rho: float, out_dtype=torch.float32,
              workspace: torch.Tensor = None, out: torch.Tensor = None, idx: torch.Tensor = None):
    """Reduced product with int8 weights: Y = A[:, I] (Bq[I, :] * scale) with A bf16 (n, d), Bq int8 (d, m)
    and scale fp32 (m,).  Returns (idx, Y)."""
    dev = _check_dev(A, Bq)
    n, d = A.shape
    d2, m = Bq.shape
    if d2 != d:
        raise ValueError("A and Bq disagree on the contraction size")
    if A.dtype != torch.bfloat16 or Bq.dtype != torch.int8 or scale.dtype != torch.float32:
        raise TypeError("A bf16, Bq int8 and scale fp32 expected")
    if A.stride(1) != 1 or Bq.stride(1) != 1 or not scale.is_contiguous() or scale.numel() != m:
        raise ValueError("unit inner strides and one scale per column of Bq expected")
    L = lib()
    kk = k(rho, d)
    if idx is None:
        idx = torch.empty(kk, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((n, m), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_matmul_w8_workspace(n, d, m, A.stride(0), float(rho)), dev)
    st = L.rmm_matmul_w8(A.data_ptr(), RMM_BF16, Bq.data_ptr(), scale.data_ptr(), n, d, m, A.stride(0), Bq.stride(0),
                         float(rho), idx.data_ptr(), out.data_ptr(), _dt(out), out.stride(0), workspace.data_ptr(),
                         workspace.numel(), _stream(dev))
    _raise(st, "rmm_matmul_w8")
    return idx, out


def workspace_bytes(op: str, n_or_heads: int, d: int, m: int) -> int:
    """rmm_workspace_bytes: a workspace size that serves every call of `op`
    with these sizes (any rho, dtype, stride or alignment)."""
    return int(lib().rmm_workspace_bytes(OPS[op], int(n_or_heads), int(d), int(m)))


def matmul_workspace(n: int, d: int, m: int, lda: int, dtype, rho: float) -> int:
    code = RMM_BF16 if dtype == torch.bfloat16 else RMM_FP32
    return int(lib().rmm_matmul_workspace(n, d, m, lda, code, float(rho)))


def qk(Q: torch.Tensor, K: torch.Tensor, rho: float, out_dtype=torch.float32, workspace: torch.Tensor = None,
       out: torch.Tensor = None, idx: torch.Tensor = None, causal: bool = False):
    """Per-head reduced Q K^T.  Q (hq, tq, dh), K (hkv, tk, dh).  Returns (idx (hq, k), S (hq, tq, tk)).
    With causal=True (rmm_qk_causal) query row r sees keys t <= r + tk - tq; later scores are -inf."""
    dev = _check_dev(Q, K)
    hq, tq, dh = Q.shape
    hkv, tk, dh2 = K.shape
    if dh2 != dh or Q.stride(2) != 1 or K.stride(2) != 1:
        raise ValueError("Q and K need the same head dim and unit inner stride")
    if Q.dtype != K.dtype:
        raise TypeError("Q and K must share a dtype")
    L = lib()
    kk = k(rho, dh)
    if idx is None:
        idx = torch.empty((hq, kk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((hq, tq, tk), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_qk_workspace(hq, tq, tk, dh, _dt(Q), float(rho)), dev)
    fn = L.rmm_qk_causal if causal else L.rmm_qk
    st = fn(Q.data_ptr(), K.data_ptr(), _dt(Q), hq, hkv, tq, tk, dh, Q.stride(0), Q.stride(1), K.stride(0),
            K.stride(1), float(rho), idx.data_ptr(), out.data_ptr(), _dt(out), workspace.data_ptr(),
            workspace.numel(), _stream(dev))
    _raise(st, "rmm_qk_causal" if causal else "rmm_qk")
    return idx, out


def qk_workspace(hq, tq, tk, dh, dtype, rho) -> int:
    code = RMM_BF16 if dtype == torch.bfloat16 else RMM_FP32
    return int(lib().rmm_qk_workspace(hq, tq, tk, dh, code, float(rho)))


def pv(P: torch.Tensor, V: torch.Tensor, rho: float, out_dtype=torch.float32, workspace: torch.Tensor = None,
       out: torch.Tensor = None, idx: torch.Tensor = None):
    """Per-head reduced P V.  P (h, tq, tk), V (hkv, tk, dv).  Returns (idx (h, k), O (h, tq, dv))."""
    dev = _check_dev(P, V)
    h, tq, tk = P.shape
    hkv, tk2, dv = V.shape
    if tk2 != tk or P.stride(2) != 1 or V.stride(2) != 1:
        raise ValueError("P key axis must match V rows; unit inner strides")
    L = lib()
    kk = k(rho, tk)
    if idx is None:
        idx = torch.empty((h, kk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((h, tq, dv), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_pv_workspace(h, tq, tk, dv, _dt(P), _dt(V), float(rho)), dev)
    st = L.rmm_pv(P.data_ptr(), _dt(P), V.data_ptr(), _dt(V), h, hkv, tq, tk, dv, P.stride(0), P.stride(1),
                  V.stride(0), V.stride(1), float(rho), idx.data_ptr(), out.data_ptr(), _dt(out),
                  workspace.data_ptr(), workspace.numel(), _stream(dev))
    _raise(st, "rmm_pv")
    return idx, out


def softmax_energy(L_: torch.Tensor, scale: float = 1.0, P: torch.Tensor = None, energy: torch.Tensor = None):
    """Row softmax of scale * logits (fp32, (h, tq, tk)) into P, with the
    column energies energy[h][j] = sum over rows of P^2.  Returns (P, energy)."""
    dev = _check_dev(L_)
    if L_.dtype != torch.float32 or L_.dim() != 3 or L_.stride(2) != 1:
        raise TypeError("logits must be fp32 (h, tq, tk) with unit inner stride")
    h, tq, tk = L_.shape
    if P is None:
        P = torch.empty((h, tq, tk), dtype=torch.float32, device=dev)
    if energy is None:
        energy = torch.empty((h, tk), dtype=torch.float32, device=dev)
    L = lib()
    ws = _ws(L.rmm_softmax_energy_workspace(h, tq, tk), dev)
    st = L.rmm_softmax_energy(L_.data_ptr(), float(scale), h, tq, tk, L_.stride(0), L_.stride(1), P.data_ptr(), P.stride(0),
                              P.stride(1), energy.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _raise(st, "rmm_softmax_energy")
    return P, energy


def softmax_select(L_: torch.Tensor, rho: float, scale: float = 1.0, P: torch.Tensor = None,
                   energy: torch.Tensor = None, idx: torch.Tensor = None):
    """rmm_softmax_select: softmax_energy and, for every head, the k = ceil(rho tk)
    key positions of largest energy (ascending).  Returns (P, energy, idx (h, k))."""
    dev = _check_dev(L_)
    if L_.dtype != torch.float32 or L_.dim() != 3 or L_.stride(2) != 1:
        raise TypeError("logits must be fp32 (h, tq, tk) with unit inner stride")
    h, tq, tk = L_.shape
    if P is None:
        P = torch.empty((h, tq, tk), dtype=torch.float32, device=dev)
    if energy is None:
        energy = torch.empty((h, tk), dtype=torch.float32, device=dev)
    L = lib()
    if idx is None:
        idx = torch.empty((h, k(rho, tk)), dtype=torch.int32, device=dev)
    ws = _ws(L.rmm_softmax_select_workspace(h, tq, tk), dev)
    st = L.rmm_softmax_select(L_.data_ptr(), float(scale), h, tq, tk, L_.stride(0), L_.stride(1), P.data_ptr(),
                              P.stride(0), P.stride(1), energy.data_ptr(), float(rho), idx.data_ptr(), ws.data_ptr(),
                              ws.numel(), _stream(dev))
    _raise(st, "rmm_softmax_select")
    return P, energy, idx


def pv_idx(P: torch.Tensor, V: torch.Tensor, idx: torch.Tensor, out_dtype=torch.float32,
           workspace: torch.Tensor = None, out: torch.Tensor = None) -> torch.Tensor:
    """rmm_pv_idx: per-head P V over given key lists idx (h, k) int32 (entries
    outside [0, tk) contribute nothing).  Returns O (h, tq, dv)."""
    dev = _check_dev(P, V, idx)
    h, tq, tk = P.shape
    hkv, tk2, dv = V.shape
    if tk2 != tk or P.stride(2) != 1 or V.stride(2) != 1:
        raise ValueError("P key axis must match V rows; unit inner strides")
    if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != h or not idx.is_contiguous():
        raise TypeError("idx must be a contiguous int32 (h, k) tensor")
    L = lib()
    kk = idx.shape[1]
    if out is None:
        out = torch.empty((h, tq, dv), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_pv_idx_workspace(h, tq, kk, dv, _dt(V)), dev)
    st = L.rmm_pv_idx(P.data_ptr(), _dt(P), V.data_ptr(), _dt(V), idx.data_ptr(), kk, h, hkv, tq, tk, dv,
                      P.stride(0), P.stride(1), V.stride(0), V.stride(1), out.data_ptr(), _dt(out),
                      workspace.data_ptr(), workspace.numel(), _stream(dev))
    _raise(st, "rmm_pv_idx")
    return out


def pv_energy(P: torch.Tensor, V: torch.Tensor, energy: torch.Tensor, rho: float, out_dtype=torch.float32,
              workspace: torch.Tensor = None, out: torch.Tensor = None, idx: torch.Tensor = None):
    """Per-head reduced P V with the key energies supplied (h, tk) fp32.
    Returns (idx (h, k), O (h, tq, dv))."""
    dev = _check_dev(P, V, energy)
    h, tq, tk = P.shape
    hkv, tk2, dv = V.shape
    if tk2 != tk or P.stride(2) != 1 or V.stride(2) != 1:
        raise ValueError("P key axis must match V rows; unit inner strides")
    if energy.dtype != torch.float32 or tuple(energy.shape) != (h, tk) or not energy.is_contiguous():
        raise TypeError("energy must be a contiguous fp32 (h, tk) tensor")
    L = lib()
    kk = k(rho, tk)
    if idx is None:
        idx = torch.empty((h, kk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((h, tq, dv), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = _ws(L.rmm_pv_energy_workspace(h, tq, tk, dv, _dt(P), _dt(V), float(rho)), dev)
    st = L.rmm_pv_energy(P.data_ptr(), _dt(P), V.data_ptr(), _dt(V), energy.data_ptr(), h, hkv, tq, tk, dv,
                         P.stride(0), P.stride(1), V.stride(0), V.stride(1), float(rho), idx.data_ptr(),
                         out.data_ptr(), _dt(out), workspace.data_ptr(), workspace.numel(), _stream(dev))
    _raise(st, "rmm_pv_energy")
    return idx, out


def pv_workspace(h, tq, tk, dv, p_dtype, v_dtype, rho) -> int:
    pc = RMM_BF16 if p_dtype == torch.bfloat16 else RMM_FP32
    vc = RMM_BF16 if v_dtype == torch.bfloat16 else RMM_FP32
    return int(lib().rmm_pv_workspace(h, tq, tk, dv, pc, vc, float(rho)))
