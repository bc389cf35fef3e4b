#!/usr/bin/env python3
"""Benchmark of the RMM hot path on one MI355X.

Default workload: the Llama-3.1-8B MLP down projection in prefill,
A 4096 x 14336 bf16 activations times B 14336 x 4096 bf16 weights, fp32 Y.
One step = one rmm_matmul call at each retention ratio 0.9, 0.7 and 0.5
(score, TopK, gather-pack, reduced GEMM) plus the rho = 1 dense product
that the speedups are measured against.  Inputs are resident in HBM before
the timed region; several copies of the inputs are rotated so that
consecutive calls do not find their operands in the 256 MB Infinity Cache.

Per-kernel times come from HIP events that the library records on its own
stream at the stage boundaries (the *_timed entry points).  Prints ONE JSON
line.

Other workloads (--workload) print the same kind of line:
  mlp_up_70b     A 2048 x 8192 @ B 8192 x 28672 (bf16), rho 0.8
  decode_qkv_8b  A 8 x 4096 @ B 4096 x 6144 (bf16), rho 0.8 (GEMV path)
  gqa_qk_8b      S = Q K^T per head, Q (32, 4096, 128), K (8, 4096, 128) bf16, rho 0.5
  attn_pv_70b    O = P V per head, P (64, 512, 8192) fp32, V (8, 8192, 128) bf16, rho 0.5
  decode_attn_8b one decode step of attention: QK^T, softmax with key energies, PV;
                 32 query heads, 8 kv heads, 8192 cached tokens, rho 0.5
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

METRIC = "RMM op latency & speedup vs own dense (rho=1) at Llama-8B shapes; MFMA/HBM %"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
STAGES = ("score", "topk", "pack", "gemm")


def _die_multi_gpu(n):
    print(json.dumps({"error": f"--gpus {n}: this benchmark measures one GPU only; the RMM path has no "
                               "multi-GPU collective (its sharding is described in the design notes)"}))
    sys.exit(2)


def _hip():
    import torch  # noqa: F401  (loads the HIP runtime librmm shares)
    lib_dir = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    h = ctypes.CDLL(lib_dir if os.path.exists(lib_dir) else "libamdhip64.so.7")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return h


class Events:
    """A pool of HIP events (timing enabled) created through the HIP runtime."""

    def __init__(self, hip, count):
        self.hip = hip
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            st = hip.hipEventCreate(ctypes.byref(e))
            if st != 0:
                raise RuntimeError(f"hipEventCreate failed: {st}")
            self.ev.append(e.value)

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b])
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return float(out.value)

    def array(self, start, n=5):
        return (ctypes.c_void_p * n)(*self.ev[start:start + n])

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def _repeat_for(min_seconds, fn, max_reps=16):
    """Runs fn until at least min_seconds of wall time have passed (at most
    max_reps times); returns (repetitions, seconds)."""
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds or reps >= max_reps:
            return reps, wall


CPU_SAMPLE_SECONDS = 10.0
LATENCY_ROUNDS = 3


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover - informational only
        pass
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return sum(int(p.get("num_threads", 1)) for p in threadpool_info() if p.get("user_api") == "blas")
    except Exception:  # pragma: no cover - informational only
        return os.cpu_count()


# ---------------------------------------------------------------------------
# workloads: each provides the call, its stage work and its oracle sample
# ---------------------------------------------------------------------------

def splits_last_wave(M: int, N: int, cus: int = 256) -> bool:
    """Whether the linear GEMM runs as two launches: 256 x 256 tiles over the
    columns that fill whole waves, then 128 x 128 tiles over the rest (the
    launcher's rule for a last wave that would fill at most half the CUs);
    used to name the kernels in the bench line."""
    tm, tn = -(-M // 256), -(-N // 256)
    t = tm * tn
    if M < 256 or N < 512 or t <= cus or t % cus == 0 or t % cus > cus // 2:
        return False
    n1 = tn - 1
    while n1 > 0 and (tm * n1) % cus:
        n1 -= 1
    return n1 > 0 and -(-M // 128) * -(-(N - 256 * n1) // 128) <= 2 * cus


class MatmulOp:
    """Linear / MLP product Y = A[:, I] B[I, :] (rmm_matmul)."""

    def __init__(self, name, A_cpu, B_cpu, rhos, desc, copies):
        import torch
        from input_adaptive_reduced_colnorm_amd import rmm
        self.rmm, self.L = rmm, rmm.lib()
        dev = torch.device("cuda:0")
        self.name, self.desc, self.rhos = name, desc, rhos
        self.A_cpu, self.B_cpu = A_cpu, B_cpu
        self.n, self.d = A_cpu.shape
        self.m = B_cpu.shape[1]
        self.copies = copies
        self.As = [A_cpu.to(dev) for _ in range(copies)]
        self.Bs = [B_cpu.to(dev) for _ in range(copies)]
        self.Y = torch.empty((self.n, self.m), dtype=torch.float32, device=dev)
        self.ks = {r: rmm.k(r, self.d) for r in rhos}
        self.idx = {r: torch.empty(self.ks[r], dtype=torch.int32, device=dev) for r in rhos}
        wsb = max(int(self.L.rmm_matmul_workspace(self.n, self.d, self.m, self.d, rmm.RMM_BF16, r)) for r in rhos)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        # the given-index calls get their own workspace, allocated here so
        # that no allocation falls inside a timed region
        wsb = max(int(self.L.rmm_matmul_idx_workspace(self.n, self.ks[r], self.m, rmm.RMM_BF16)) for r in rhos)
        self.ws_idx = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        self.decode = self.n <= 16

    def call(self, c, rho, sh, events=None):
        n, d, m, L, rmm = self.n, self.d, self.m, self.L, self.rmm
        args = [self.As[c].data_ptr(), self.Bs[c].data_ptr(), rmm.RMM_BF16, n, d, m, d, m, float(rho),
                self.idx[rho].data_ptr(), self.Y.data_ptr(), rmm.RMM_FP32, m, self.ws.data_ptr(), self.ws.numel(), sh]
        st = L.rmm_matmul(*args) if events is None else L.rmm_matmul_timed(*args, events)
        if st != 0:
            raise RuntimeError(f"rmm_matmul: {rmm.status_str(st)}")

    def call_idx(self, c, rho, sh):
        """The product over the index set the last call at this rho selected
        (rmm_matmul_idx: the reuse of one selection for another projection)."""
        n, d, m, L, rmm = self.n, self.d, self.m, self.L, self.rmm
        st = L.rmm_matmul_idx(self.As[c].data_ptr(), self.Bs[c].data_ptr(), rmm.RMM_BF16, n, d, m, d, m,
                              self.idx[rho].data_ptr(), self.ks[rho], self.Y.data_ptr(), rmm.RMM_FP32, m,
                              self.ws_idx.data_ptr(), self.ws_idx.numel(), sh)
        if st != 0:
            raise RuntimeError(f"rmm_matmul_idx: {rmm.status_str(st)}")

    def stage_work(self, rho):
        """Algorithmic work per stage: (kind, amount) with kind 'B' bytes or 'F' flops."""
        n, d, m, k = self.n, self.d, self.m, self.ks[rho]
        if self.decode:
            # rows of up to 8192 columns: every GEMV workgroup ranks the
            # columns of A itself, so the GEMV stage holds the selection;
            # wider rows select in one workgroup first
            w = {"gemm": ("B", k * m * 2)}
            if k < d and d > 8192:
                w["score"] = ("B", n * d * 2)
            return w
        w = {"gemm": ("F", 2.0 * n * k * m)}
        if k < d:
            w["score"] = ("B", n * d * 2)
            if self.fused(rho):
                # one launch ranks the keys and gathers: whole rows of A in,
                # the kept columns out (stage events 1 -> 2 bracket it)
                w["topk"] = ("B", n * d * 2 + n * k * 2)
            else:
                w["pack"] = ("B", 2 * n * k * 2)
        return w

    def fused(self, rho):
        """Whether the prefill product at this rho ranks and gathers in one
        launch (the library's rule for a contiguous bf16 A: at most 15360
        columns, whole 16-byte row pieces)."""
        return (not self.decode) and self.ks[rho] < self.d and self.d <= 15360 and self.d % 8 == 0

    def roofline_stage(self):
        return "gemm"

    def roofline_kernel(self):
        if self.decode:
            return ("gemv_rank_kernel + gemv_reduce_kernel (each workgroup ranks the columns of A while the first "
                    "rows of its slice of B stream in, then reads the kept rows; the slices added in order)")
        if splits_last_wave(self.n, self.m):
            return ("gemm_bf16_kernel<256,256,kmajor,gather> over the columns that fill whole waves + "
                    "gemm_bf16_kernel<128,128,kmajor,gather> over the rest (reduced GEMM, two launches)")
        return "gemm_bf16_kernel<256,256,kmajor,gather> (reduced GEMM)"

    def traffic_ref(self):
        return None if self.decode else f"gemm_bf16_kernel_{self.name}_traffic.json"

    def shape(self):
        return {"shape": self.desc}

    def cpu_baseline(self):
        """The oracle as it stands, on the whole step (every rho, every row)."""
        import numpy as np
        from oracle import rmm_oracle as O
        A = self.A_cpu.float().numpy()
        B = self.B_cpu.float().numpy()
        rows = None
        if self.n * self.d * self.m > 4096 * 14336 * 4096:
            rows = np.arange(1024)        # bound the sample for larger shapes
        reps, wall = _repeat_for(CPU_SAMPLE_SECONDS, lambda: [O.matmul(A, B, rho, rows=rows) for rho in self.rhos])
        scale = 1 if rows is None else self.n / len(rows)
        ops = reps * len(self.rhos) / (wall * scale)
        what = "every row" if rows is None else f"rows 0..{len(rows) - 1} of {self.n} (product), scaled by {scale:g}x"
        return {"value": ops, "unit": "RMM ops/s", "cores": _blas_threads(), "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
                "kind": "oracle",
                "sample": (f"fp64 oracle (scoring, stable-sort TopK, gather, product) for one call per rho in "
                           f"{list(self.rhos)} over {what}, {reps} repetitions; {wall:.1f} s of CPU work"),
                "stages_ms": self._cpu_stages(O, A, B, rows)}

    def _cpu_stages(self, O, A, B, rows):
        """One pass per rho of the oracle's steps, each timed on its own (ms):
        the column energies (O.col_energy), the stable-sort selection
        (O.select minus its energies), the gather of A[:, I] and B[I, :]
        and the fp64 product of the gathered slices (the two halves of the
        oracle's product line)."""
        import numpy as np
        A64 = np.asarray(A, dtype=np.float64)
        B64 = np.asarray(B, dtype=np.float64)
        out = {}
        for rho in self.rhos:
            t0 = time.perf_counter()
            O.col_energy(A64)
            t1 = time.perf_counter()
            idx, _ = O.select(A64, rho)
            t2 = time.perf_counter()
            Ar = A64 if rows is None else A64[rows]
            Ag, Bg = Ar[:, idx], B64[idx, :]
            t3 = time.perf_counter()
            Ag @ Bg
            t4 = time.perf_counter()
            sc = 1 if rows is None else self.n / len(rows)
            out[str(rho)] = {"norms": round(1e3 * (t1 - t0), 2), "stable_sort": round(1e3 * max(0.0, (t2 - t1) - (t1 - t0)), 2),
                             "gather": round(1e3 * (t3 - t2) * sc, 2), "dgemm_fp64": round(1e3 * (t4 - t3) * sc, 2)}
        return out


class MatmulW8Op(MatmulOp):
    """Linear product with int8 weights and a scale per output column,
    Y = A[:, I] (Bq[I, :] diag(scale)) (rmm_matmul_w8)."""

    def __init__(self, name, A_cpu, Bq_cpu, scale_cpu, rhos, desc, copies):
        import torch
        from input_adaptive_reduced_colnorm_amd import rmm
        self.rmm, self.L = rmm, rmm.lib()
        dev = torch.device("cuda:0")
        self.name, self.desc, self.rhos = name, desc, rhos
        self.A_cpu, self.Bq_cpu, self.scale_cpu = A_cpu, Bq_cpu, scale_cpu
        self.n, self.d = A_cpu.shape
        self.m = Bq_cpu.shape[1]
        self.copies = copies
        self.As = [A_cpu.to(dev) for _ in range(copies)]
        self.Bqs = [Bq_cpu.to(dev) for _ in range(copies)]
        self.scale = scale_cpu.to(dev)
        self.Y = torch.empty((self.n, self.m), dtype=torch.float32, device=dev)
        self.ks = {r: rmm.k(r, self.d) for r in rhos}
        self.idx = {r: torch.empty(self.ks[r], dtype=torch.int32, device=dev) for r in rhos}
        wsb = max(int(self.L.rmm_matmul_w8_workspace(self.n, self.d, self.m, self.d, r)) for r in rhos)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        self.decode = self.n <= 16

    call_idx = None   # no int8 variant of the given-index product

    def call(self, c, rho, sh, events=None):
        n, d, m, L, rmm = self.n, self.d, self.m, self.L, self.rmm
        args = [self.As[c].data_ptr(), rmm.RMM_BF16, self.Bqs[c].data_ptr(), self.scale.data_ptr(), n, d, m, d, m,
                float(rho), self.idx[rho].data_ptr(), self.Y.data_ptr(), rmm.RMM_FP32, m, self.ws.data_ptr(),
                self.ws.numel(), sh]
        st = L.rmm_matmul_w8(*args) if events is None else L.rmm_matmul_w8_timed(*args, events)
        if st != 0:
            raise RuntimeError(f"rmm_matmul_w8: {rmm.status_str(st)}")

    def stage_work(self, rho):
        n, d, m, k = self.n, self.d, self.m, self.ks[rho]
        if self.decode:
            w = {"gemm": ("B", k * m * 1)}
            if k < d and d > 8192:
                w["score"] = ("B", n * d * 2)
            return w
        w = {"gemm": ("F", 2.0 * n * k * m)}
        if k < d:
            w["score"] = ("B", n * d * 2)
            if self.fused(rho):
                # one launch ranks the keys and gathers: whole rows of A in,
                # the kept columns out (stage events 1 -> 2 bracket it)
                w["topk"] = ("B", n * d * 2 + n * k * 2)
            else:
                w["pack"] = ("B", 2 * n * k * 2)
        return w

    def roofline_kernel(self):
        if self.decode:
            return ("gemv_rank_kernel<bf16 A, int8 B> + gemv_reduce_kernel (each workgroup ranks the columns of A "
                    "while the first rows of its slice stream in, then reads the kept int8 rows of B; the slices "
                    "added in order)")
        if splits_last_wave(self.n, self.m):
            return ("gemm_bf16_kernel<256,256,kmajor,gather,int8 B> over the columns that fill whole waves + "
                    "gemm_bf16_kernel<128,128,kmajor,gather,int8 B> over the rest (reduced GEMM, two launches)")
        return "gemm_bf16_kernel<256,256,kmajor,gather,int8 B> (reduced GEMM)"

    def traffic_ref(self):
        return None

    extra_key = "bf16_weights_context"

    def extra(self, args, sh):
        """The same call with the weights dequantised to bf16 (rmm_matmul), at
        each rho, for the int8-over-bf16 comparison."""
        import torch
        rmm, L = self.rmm, self.L
        dev = self.Y.device
        Bb = [(self.Bqs[c].float() * self.scale[None, :]).to(torch.bfloat16) for c in range(self.copies)]
        wsb = max(int(L.rmm_matmul_workspace(self.n, self.d, self.m, self.d, rmm.RMM_BF16, r)) for r in self.rhos)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)
        out = {}
        for rho in self.rhos:
            def one(c):
                st = L.rmm_matmul(self.As[c].data_ptr(), Bb[c].data_ptr(), rmm.RMM_BF16, self.n, self.d, self.m,
                                  self.d, self.m, float(rho), self.idx[rho].data_ptr(), self.Y.data_ptr(),
                                  rmm.RMM_FP32, self.m, ws.data_ptr(), ws.numel(), sh)
                if st != 0:
                    raise RuntimeError(f"rmm_matmul: {rmm.status_str(st)}")
            one(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                one(i % self.copies)
            e1.record(stream)
            torch.cuda.synchronize()
            out[str(rho)] = round(e0.elapsed_time(e1) / args.steps * 1e3, 2)
        del Bb
        return {"bf16_weights_latency_us": out,
                "note": "rmm_matmul on the same weights dequantised to bf16 (twice the weight bytes)"}

    def cpu_baseline(self):
        import numpy as np
        from oracle import rmm_oracle as O
        A = self.A_cpu.float().numpy()
        Bq = self.Bq_cpu.numpy()
        sc = self.scale_cpu.numpy()
        rows = None if self.n <= 1024 else np.arange(1024)
        reps, wall = _repeat_for(CPU_SAMPLE_SECONDS,
                                 lambda: [O.matmul_w8(A, Bq, sc, rho, rows=rows) for rho in self.rhos])
        scale = 1 if rows is None else self.n / len(rows)
        what = "every row" if rows is None else f"rows 0..{len(rows) - 1} of {self.n} (product), scaled by {scale:g}x"
        return {"value": reps * len(self.rhos) / (wall * scale), "unit": "RMM ops/s", "cores": _blas_threads(),
                "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(), "kind": "oracle",
                "sample": (f"fp64 oracle with int8 weights for one call per rho in {list(self.rhos)} over {what}, "
                           f"{reps} repetitions; {wall:.1f} s of CPU work")}


class QkOp:
    """Per-head attention scores S_h = Q_h[:, I_h] K_g(h)[:, I_h]^T (rmm_qk)."""

    def __init__(self, name, Q_cpu, K_cpu, rhos, desc, copies):
        import torch
        from input_adaptive_reduced_colnorm_amd import rmm
        self.rmm, self.L = rmm, rmm.lib()
        dev = torch.device("cuda:0")
        self.name, self.desc, self.rhos, self.copies = name, desc, rhos, copies
        self.Q_cpu, self.K_cpu = Q_cpu, K_cpu
        self.hq, self.tq, self.dh = Q_cpu.shape
        self.hkv, self.tk, _ = K_cpu.shape
        self.Qs = [Q_cpu.to(dev) for _ in range(copies)]
        self.Ks = [K_cpu.to(dev) for _ in range(copies)]
        self.S = torch.empty((self.hq, self.tq, self.tk), dtype=torch.float32, device=dev)
        self.ks = {r: rmm.k(r, self.dh) for r in rhos}
        self.idx = {r: torch.empty((self.hq, self.ks[r]), dtype=torch.int32, device=dev) for r in rhos}
        wsb = max(int(self.L.rmm_qk_workspace(self.hq, self.tq, self.tk, self.dh, rmm.RMM_BF16, r)) for r in rhos)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def call(self, c, rho, sh, events=None):
        hq, tq, tk, dh, L, rmm = self.hq, self.tq, self.tk, self.dh, self.L, self.rmm
        args = [self.Qs[c].data_ptr(), self.Ks[c].data_ptr(), rmm.RMM_BF16, hq, self.hkv, tq, tk, dh, tq * dh, dh,
                tk * dh, dh, float(rho), self.idx[rho].data_ptr(), self.S.data_ptr(), rmm.RMM_FP32,
                self.ws.data_ptr(), self.ws.numel(), sh]
        st = L.rmm_qk(*args) if events is None else L.rmm_qk_timed(*args, events)
        if st != 0:
            raise RuntimeError(f"rmm_qk: {rmm.status_str(st)}")

    extra_key = "causal_scores"

    def extra(self, args, sh):
        """Causal scores (rmm_qk_causal: keys after the query position get
        -inf) beside the unmasked call, at each rho, back to back outside the
        stepped loop."""
        import torch
        if self.tq > self.tk:
            return None
        dev = self.Qs[0].device
        stream = torch.cuda.current_stream(dev)
        out = {}
        for rho in self.rhos:
            def run(c, fn):
                st = fn(self.Qs[c].data_ptr(), self.Ks[c].data_ptr(), self.rmm.RMM_BF16, self.hq, self.hkv, self.tq,
                        self.tk, self.dh, self.tq * self.dh, self.dh, self.tk * self.dh, self.dh, float(rho),
                        self.idx[rho].data_ptr(), self.S.data_ptr(), self.rmm.RMM_FP32, self.ws.data_ptr(),
                        self.ws.numel(), sh)
                if st != 0:
                    raise RuntimeError(f"rmm_qk: {self.rmm.status_str(st)}")
            us = {}
            for name, fn in (("causal", self.L.rmm_qk_causal), ("unmasked", self.L.rmm_qk)):
                run(0, fn)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(args.steps):
                    run(i % self.copies, fn)
                e1.record(stream)
                torch.cuda.synchronize()
                us[name] = e0.elapsed_time(e1) / args.steps * 1e3
            out[str(rho)] = {"causal_latency_us": round(us["causal"], 2),
                             "unmasked_latency_us": round(us["unmasked"], 2)}
        out["note"] = ("the causal call writes the same S bytes (-inf above the diagonal); with this many tiles "
                       "both run the persistent score kernel, which multiplies every tile since the store is the "
                       "cost")
        return out

    def stage_work(self, rho):
        hq, hkv, tq, tk, dh, k = self.hq, self.hkv, self.tq, self.tk, self.dh, self.ks[rho]
        s_bytes = hq * tq * tk * 4
        if k == dh:   # dense: Q and K read in place, S written
            return {"gemm": ("B", s_bytes + hq * tq * dh * 2 + hkv * tk * dh * 2)}
        w = {"score": ("B", hq * tq * dh * 2),
             "gemm": ("B", s_bytes + (hq * tq * k + hq * tk * k) * 2)}
        if self.fused(rho):
            # one launch ranks each head's features and gathers Q and K:
            # whole rows of Q and of the kv heads' K in, both panels out
            w["topk"] = ("B", hq * tq * dh * 2 + hkv * tk * dh * 2 + (hq * tq * k + hq * tk * k) * 2)
        else:
            w["pack"] = ("B", 2 * (hq * tq * k + hq * tk * k) * 2)
        return w

    def fused(self, rho):
        """Whether the call ranks the features and gathers Q and K in one
        launch (the library's rule for contiguous bf16 heads of at most 256
        features in whole 16-byte pieces)."""
        return self.ks[rho] < self.dh and self.dh <= 256 and self.dh % 8 == 0

    def roofline_stage(self):
        return "gemm"

    def roofline_kernel(self):
        return ("gemm_nmajor_persistent_kernel (batched per-head QK^T, one workgroup per CU walking the "
                "256x256 score tiles, fp32 S store)")

    def traffic_ref(self):
        return None

    def shape(self):
        return {"shape": self.desc}

    def cpu_baseline(self):
        import numpy as np
        from oracle import rmm_oracle as O
        Q = self.Q_cpu.float().numpy()
        K = self.K_cpu.float().numpy()
        heads = list(range(0, self.hq, 4))          # 8 of 32 query heads
        reps, wall = _repeat_for(CPU_SAMPLE_SECONDS, lambda: [O.qk(Q, K, rho, heads=heads) for rho in self.rhos])
        scale = self.hq / len(heads)
        return {"value": reps * len(self.rhos) / (wall * scale), "unit": "RMM ops/s", "cores": _blas_threads(),
                "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(), "kind": "oracle",
                "sample": (f"fp64 oracle qk for query heads {heads[0]}, {heads[1]}, ... (every 4th, "
                           f"{len(heads)} of {self.hq}) at each rho in {list(self.rhos)}, scaled by {scale:g}x, "
                           f"{reps} repetitions; {wall:.1f} s of CPU work")}


class PvOp:
    """Per-head attention output O_h = P_h[:, I_h] V_g(h)[I_h, :] (rmm_pv)."""

    def __init__(self, name, P_cpu, V_cpu, rhos, desc, copies, L_cpu=None):
        import torch
        from input_adaptive_reduced_colnorm_amd import rmm
        self.rmm, self.L = rmm, rmm.lib()
        dev = torch.device("cuda:0")
        self.name, self.desc, self.rhos, self.copies = name, desc, rhos, copies
        self.P_cpu, self.V_cpu, self.L_cpu = P_cpu, V_cpu, L_cpu
        self.h, self.tq, self.tk = P_cpu.shape
        self.hkv, _, self.dv = V_cpu.shape
        self.Ps = [P_cpu.to(dev) for _ in range(copies)]
        self.Vs = [V_cpu.to(dev) for _ in range(copies)]
        self.O = torch.empty((self.h, self.tq, self.dv), dtype=torch.float32, device=dev)
        self.ks = {r: rmm.k(r, self.tk) for r in rhos}
        self.idx = {r: torch.empty((self.h, self.ks[r]), dtype=torch.int32, device=dev) for r in rhos}
        wsb = max(int(self.L.rmm_pv_workspace(self.h, self.tq, self.tk, self.dv, rmm.RMM_FP32, rmm.RMM_BF16, r))
                  for r in rhos)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def call(self, c, rho, sh, events=None):
        h, tq, tk, dv, L, rmm = self.h, self.tq, self.tk, self.dv, self.L, self.rmm
        args = [self.Ps[c].data_ptr(), rmm.RMM_FP32, self.Vs[c].data_ptr(), rmm.RMM_BF16, h, self.hkv, tq, tk, dv,
                tq * tk, tk, tk * dv, dv, float(rho), self.idx[rho].data_ptr(), self.O.data_ptr(), rmm.RMM_FP32,
                self.ws.data_ptr(), self.ws.numel(), sh]
        st = L.rmm_pv(*args) if events is None else L.rmm_pv_timed(*args, events)
        if st != 0:
            raise RuntimeError(f"rmm_pv: {rmm.status_str(st)}")

    def extra(self, args, sh):
        """Producer-side scoring: the softmax pass over the logits writes P and
        the key energies; PV then runs on the supplied energies (no scoring
        pass over P).  Times both, back to back, outside the stepped loop."""
        import torch
        rmm, L = self.rmm, self.L
        if self.L_cpu is None:
            return None
        dev = self.Ps[0].device
        Ld = self.L_cpu.to(dev)
        Pout = torch.empty_like(self.Ps[0])
        E = torch.empty((self.h, self.tk), dtype=torch.float32, device=dev)
        ws = torch.empty(max(int(L.rmm_softmax_energy_workspace(self.h, self.tq, self.tk)), 256), dtype=torch.uint8,
                         device=dev)

        def producer():
            st = L.rmm_softmax_energy(Ld.data_ptr(), 1.0, self.h, self.tq, self.tk, self.tq * self.tk, self.tk,
                                      Pout.data_ptr(), self.tq * self.tk, self.tk, E.data_ptr(), ws.data_ptr(),
                                      ws.numel(), sh)
            if st != 0:
                raise RuntimeError(f"rmm_softmax_energy: {rmm.status_str(st)}")

        rho = min(self.rhos)
        wsp = torch.empty(max(int(L.rmm_pv_energy_workspace(self.h, self.tq, self.tk, self.dv, rmm.RMM_FP32,
                                                             rmm.RMM_BF16, rho)), 256), dtype=torch.uint8, device=dev)

        def pv_e(c):
            st = L.rmm_pv_energy(self.Ps[c].data_ptr(), rmm.RMM_FP32, self.Vs[c].data_ptr(), rmm.RMM_BF16,
                                 E.data_ptr(), self.h, self.hkv, self.tq, self.tk, self.dv, self.tq * self.tk, self.tk,
                                 self.tk * self.dv, self.dv, float(rho), self.idx[rho].data_ptr(), self.O.data_ptr(),
                                 rmm.RMM_FP32, wsp.data_ptr(), wsp.numel(), sh)
            if st != 0:
                raise RuntimeError(f"rmm_pv_energy: {rmm.status_str(st)}")

        def timed(fn, n):
            stream = torch.cuda.current_stream(dev)
            fn(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                fn(i % self.copies)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n * 1e3

        prod_us = timed(lambda c: producer(), args.steps)
        pv_us = timed(pv_e, args.steps)
        prod_bytes = 2 * self.h * self.tq * self.tk * 4
        return {"rho": rho,
                "softmax_energy_us": round(prod_us, 2),
                "softmax_energy_gbs": round(prod_bytes / (prod_us * 1e-6) / 1e9, 1),
                "pv_energy_latency_us": round(pv_us, 2),
                "note": ("rmm_softmax_energy writes P (fp32) and the key energies from the logits; rmm_pv_energy "
                         "then selects on those energies and never scores P; compare pv_energy_latency_us with "
                         "latency_us['1.0']")}

    def masked(self, rho):
        """The library runs PV over all key positions of P in place (dropped
        rows of V read as zeros) when at least one key in eight is kept."""
        return self.ks[rho] * 8 >= self.tk and self.tk % 64 == 0

    def stage_work(self, rho):
        h, tq, tk, dv, k = self.h, self.tq, self.tk, self.dv, self.ks[rho]
        o_bytes = h * tq * dv * 4
        if k == tk:   # dense: fp32 P and V read in place
            return {"gemm": ("B", h * tq * tk * 4 + self.hkv * tk * dv * 2 + o_bytes)}
        score = ("B", h * tq * tk * 4)
        if self.masked(rho):
            # P read in place once more, kept rows of V, O written
            return {"score": score, "gemm": ("B", h * tq * tk * 4 + h * k * dv * 2 + o_bytes)}
        return {"score": score,
                "pack": ("B", h * tq * k * 4 + h * tq * k * 2),
                "gemm": ("B", h * tq * k * 2 + h * k * dv * 2 + o_bytes)}

    def roofline_stage(self):
        return None   # the slowest stage of the reduced op

    def roofline_kernel(self):
        masked = all(self.masked(r) for r in self.rhos if r < 1.0)
        gemm = ("gemm_bf16_kernel<128,128,kmajor,gather,fp32 A> (per-head PV over all keys of P, dropped V rows "
                "masked)" if masked else "gemm_bf16_kernel<128,128,kmajor,gather> (per-head PV on packed P)")
        return {"score": "colnorm_kernel<fp32> (column energies of P)", "pack": "pack_kernel<fp32> (kept columns of P)",
                "gemm": gemm}

    def traffic_ref(self):
        return None

    def shape(self):
        return {"shape": self.desc}

    def cpu_baseline(self):
        import numpy as np
        from oracle import rmm_oracle as O
        P = self.P_cpu.numpy()
        V = self.V_cpu.float().numpy()
        heads = list(range(0, self.h, 4))           # 16 of 64 heads
        reps, wall = _repeat_for(CPU_SAMPLE_SECONDS, lambda: [O.pv(P, V, rho, heads=heads) for rho in self.rhos])
        scale = self.h / len(heads)
        return {"value": reps * len(self.rhos) / (wall * scale), "unit": "RMM ops/s", "cores": _blas_threads(),
                "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(), "kind": "oracle",
                "sample": (f"fp64 oracle pv for heads {heads[0]}, {heads[1]}, ... (every 4th, {len(heads)} of "
                           f"{self.h}) at each rho in {list(self.rhos)}, scaled by {scale:g}x, "
                           f"{reps} repetitions; {wall:.1f} s of CPU work")}


# ---------------------------------------------------------------------------

ROOT = os.path.dirname(os.path.abspath(__file__))


def measured_traffic(op):
    """HBM bytes per launch of the roofline kernel from the committed counter
    runs (profiles/), or None when there are none or the kernel source has
    changed since they were taken."""
    ref = op.traffic_ref()
    if ref is None:
        return None, None
    path = os.path.join(ROOT, "profiles", ref)
    if not os.path.exists(path):
        return None, None
    import hashlib
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec["kernel_source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["kernel_source_sha256"]:
        return None, "stale: " + ref
    return rec["hbm_bytes_per_launch"]["total"], ref


def _rate(kind, amount, us):
    if kind == "F":
        v = amount / (us * 1e-6) / 1e12
        return {"tflops": round(v, 1), "mfma_frac": round(v / PEAK_BF16_TFLOPS, 4)}
    v = amount / (us * 1e-6) / 1e9
    return {"gbs": round(v, 1), "hbm_frac": round(v / PEAK_HBM_GBS, 4)}


def run(args, op):
    import torch

    hip = _hip()
    stream = torch.cuda.current_stream(torch.device("cuda:0"))
    sh = stream.cuda_stream
    rhos = op.rhos
    nops = len(rhos)
    copies = op.copies

    for step in range(args.warmup):
        for j, rho in enumerate(rhos):
            op.call((step * nops + j) % copies, rho, sh)
    torch.cuda.synchronize()

    # timed region: K steps; barrier (single process) + device sync on both sides
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for step in range(args.steps):
        for j, rho in enumerate(rhos):
            op.call((step * nops + j) % copies, rho, sh)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)

    # op latency per rho: back-to-back calls between two events (no events
    # between calls: an event record costs a few microseconds of GPU time).
    # The clock drifts while the chip warms up and under sustained power
    # limits, so the blocks run in three rounds, in alternating rho order,
    # and each rho reports its median block
    samples = {rho: [] for rho in rhos}
    for rd in range(LATENCY_ROUNDS):
        for rho in (rhos if rd % 2 == 0 else tuple(reversed(rhos))):
            j = rhos.index(rho)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for it in range(args.steps):
                op.call((it + j) % copies, rho, sh)
            e1.record(stream)
            torch.cuda.synchronize()
            samples[rho].append(e0.elapsed_time(e1) / args.steps * 1e3)
    op_us = {rho: statistics.median(v) for rho, v in samples.items()}

    # the same products over the index sets just selected (selection reused)
    reuse_us = {}
    if getattr(op, "call_idx", None):
        for j, rho in enumerate(rhos):
            if rho >= 1.0:
                continue
            op.call(j % copies, rho, sh)   # the index set of this rho
            op.call_idx(j % copies, rho, sh)   # untimed first call
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for it in range(args.steps):
                op.call_idx((it + j) % copies, rho, sh)
            e1.record(stream)
            torch.cuda.synchronize()
            reuse_us[str(rho)] = round(e0.elapsed_time(e1) / args.steps * 1e3, 2)

    # per-kernel durations: the same calls with stage events recorded by the
    # library on the stream the kernels run on
    evs = Events(hip, 5 * args.stage_iters * nops)
    names = getattr(op, "stage_names", STAGES)
    stages = {r: {s: [] for s in names + ("op",)} for r in rhos}
    slot = 0
    for it in range(args.stage_iters):
        for j, rho in enumerate(rhos):
            op.call((it * nops + j) % copies, rho, sh, evs.array(5 * slot))
            slot += 1
    torch.cuda.synchronize()
    slot = 0
    for it in range(args.stage_iters):
        for rho in rhos:
            b = 5 * slot
            for i, s in enumerate(names):
                stages[rho][s].append(evs.ms(b + i, b + i + 1))
            stages[rho]["op"].append(evs.ms(b, b + 4))
            slot += 1
    evs.close()
    mean = {r: {s: statistics.fmean(v) * 1e3 for s, v in stages[r].items()} for r in rhos}   # us

    dense_r = 1.0 if 1.0 in rhos else None
    speed = {str(r): round(op_us[dense_r] / op_us[r], 4) for r in rhos if dense_r is not None and r != dense_r}
    per_kernel = {}
    for r in rhos:
        row = {}
        work = op.stage_work(r)
        for s in names:
            if s in work or (s == "topk" and "score" in work):
                row[f"{s}_us"] = round(mean[r][s], 2)
                if s in work:
                    for key, v in _rate(*work[s], mean[r][s]).items():
                        row[f"{s}_{key}"] = v
        fused = getattr(op, "fused", None) and op.fused(r)
        if fused:
            # the TopK stage is the fused ranking + gather launch
            row = {(f"select_pack{k[4:]}" if k.startswith("topk") else k): v for k, v in row.items()}
            sel_us = mean[r]["score"] + mean[r]["topk"]
            row["selection_gather_us"] = round(sel_us, 2)
            for key, v in _rate("B", work["score"][1] + work["topk"][1], sel_us).items():
                row[f"selection_gather_{key}"] = v
        elif "score" in work and work["score"][0] == "B" and "topk" in names:
            # the whole selection (energies + TopK) against the bytes of A it reads
            sel_us = mean[r]["score"] + mean[r]["topk"]
            row["selection_us"] = round(sel_us, 2)
            for key, v in _rate("B", work["score"][1], sel_us).items():
                row[f"selection_{key}"] = v
        per_kernel[str(r)] = row

    # bandwidth-bound stages also against the rate a plain copy reaches (the
    # practical ceiling beside the datasheet 8 TB/s)
    measured = hbm_copy_gbs() if any(k.endswith("_gbs") for row in per_kernel.values() for k in row) else None
    if measured:
        for row in per_kernel.values():
            for key in [k for k in row if k.endswith("_gbs")]:
                row[key[:-4] + "_frac_of_measured_copy"] = round(row[key] / measured, 4)

    # roofline of the dominant kernel of the reduced op (mean over its launches)
    red = [r for r in rhos if r != dense_r]
    stage = op.roofline_stage()
    if stage is None:
        stage = max((s for s in names if s in op.stage_work(red[0])), key=lambda s: sum(mean[r][s] for r in red))
    kinds = {op.stage_work(r)[stage][0] for r in red}
    assert len(kinds) == 1
    kind = kinds.pop()
    tot_s = sum(mean[r][stage] * 1e-6 for r in red)
    tot_w = sum(op.stage_work(r)[stage][1] for r in red)
    kname = op.roofline_kernel()
    if isinstance(kname, dict):
        kname = kname[stage]
    if kind == "F":
        achieved = tot_w / tot_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "per_launch_flops": {str(r): op.stage_work(r)[stage][1] for r in red}}
    else:
        achieved = tot_w / tot_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                    "per_launch_bytes": {str(r): op.stage_work(r)[stage][1] for r in red}}
    roofline = {"kernel": f"{kname}, stage '{stage}', mean over rho in {red}", **roofline,
                "avg_launch_us": round(tot_s / len(red) * 1e6, 2)}
    traffic, src = measured_traffic(op)
    roofline["traffic"] = traffic
    roofline["traffic_source"] = src
    if roofline["bound"] == "hbm":
        # the datasheet peak above; beside it the rate a plain copy reaches
        measured = measured or hbm_copy_gbs()
        roofline["measured_copy_gbs"] = measured
        roofline["frac_of_measured_copy"] = round(roofline["achieved"] / measured, 4)

    extra = op.extra(args, sh) if hasattr(op, "extra") else None

    line = {
        "metric": METRIC,
        "value": round(nops * args.steps / (ms_total * 1e-3), 2),
        "unit": "RMM ops/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": op.name, **op.shape(), "rhos": list(rhos),
                   "k": {str(r): op.ks[r] for r in rhos}, "copies_rotated": copies,
                   "score_separation": "every neighbouring pair" if args.strict_adjacent else "selection boundaries"},
        "latency_us": {str(r): round(op_us[r], 2) for r in rhos},
        "latency_note": "per-op mean of back-to-back calls; kernel times below come from stage events",
        "speedup_vs_dense": speed,
        "given_index_latency_us": reuse_us or None,
        "given_index_note": ("rmm_matmul_idx over the set each rho selected (pack + GEMM, no scoring or TopK): "
                             "the cost of a projection that reuses another's selection") if reuse_us else None,
        "kernels": per_kernel,
        "measured_copy_gbs": measured,
        "roofline": roofline,
    }
    if extra:
        line[getattr(op, "extra_key", "producer_side_scoring")] = extra
    return line


def hbm_copy_gbs():
    """Measured HBM rate of a plain 1 GiB device-to-device copy (bytes read
    plus bytes written per second), as the practical ceiling beside the
    datasheet 8 TB/s."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 5 * 1e3
    del src, dst
    return round(2 * (1 << 30) / (us * 1e-6) / 1e9, 1)


def hipblaslt_context(op):
    """hipBLASLt dense time at the same shape (bf16 output), as context only."""
    import torch
    if not isinstance(op, MatmulOp) or not hasattr(op, "Bs"):
        return None
    Ad, Bd = op.As[0], op.Bs[0]
    for _ in range(3):
        torch.matmul(Ad, Bd)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(Ad, Bd)
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) / 10 * 1e3, 1)


class DecodeAttnOp:
    """One decode step of attention per layer (one query per head over a KV
    cache): rmm_qk (features of q kept, streaming pass over K), the softmax
    of the scores scaled by 1/sqrt(head dim) that also ranks the key
    energies and writes the kept lists (rmm_softmax_select), and rmm_pv_idx
    (a GEMV per head over the kept V rows).  The dense step (rho = 1) runs
    rmm_softmax_energy and rmm_pv_energy, which keep every key."""

    stage_names = ("qk", "softmax", "none", "pv")

    def __init__(self, name, Q_cpu, K_cpu, V_cpu, rhos, desc, copies, hip):
        import torch
        from input_adaptive_reduced_colnorm_amd import rmm
        self.rmm, self.L, self.hip = rmm, rmm.lib(), hip
        dev = torch.device("cuda:0")
        self.name, self.desc, self.rhos, self.copies = name, desc, rhos, copies
        self.hq, self.tq, self.dh = Q_cpu.shape
        self.hkv, self.tk, _ = K_cpu.shape
        self.dv = V_cpu.shape[2]
        self.Qs = [Q_cpu.to(dev) for _ in range(copies)]
        self.Ks = [K_cpu.to(dev) for _ in range(copies)]
        self.Vs = [V_cpu.to(dev) for _ in range(copies)]
        self.S = torch.empty((self.hq, self.tq, self.tk), dtype=torch.float32, device=dev)
        self.P = torch.empty_like(self.S)
        self.E = torch.empty((self.hq, self.tk), dtype=torch.float32, device=dev)
        self.O = torch.empty((self.hq, self.tq, self.dv), dtype=torch.float32, device=dev)
        self.ks = {r: rmm.k(r, self.tk) for r in rhos}       # kept keys (PV)
        self.kf = {r: rmm.k(r, self.dh) for r in rhos}       # kept features (QK)
        self.iq = {r: torch.empty((self.hq, self.kf[r]), dtype=torch.int32, device=dev) for r in rhos}
        self.ip = {r: torch.empty((self.hq, self.ks[r]), dtype=torch.int32, device=dev) for r in rhos}
        L = self.L
        wq = max(int(L.rmm_qk_workspace(self.hq, self.tq, self.tk, self.dh, rmm.RMM_BF16, r)) for r in rhos)
        ws = max(int(L.rmm_softmax_energy_workspace(self.hq, self.tq, self.tk)), 1)
        wp = max(int(L.rmm_pv_energy_workspace(self.hq, self.tq, self.tk, self.dv, rmm.RMM_FP32, rmm.RMM_BF16, r))
                 for r in rhos)
        ws = max(ws, max(int(L.rmm_softmax_select_workspace(self.hq, self.tq, self.tk)) for r in rhos))
        wp = max(wp, max(int(L.rmm_pv_idx_workspace(self.hq, self.tq, self.ks[r], self.dv, rmm.RMM_BF16))
                         for r in rhos))
        self.wsq = torch.empty(max(wq, 256), dtype=torch.uint8, device=dev)
        self.wss = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.wsp = torch.empty(max(wp, 256), dtype=torch.uint8, device=dev)

    def call(self, c, rho, sh, events=None):
        rmm, L = self.rmm, self.L
        hq, hkv, tq, tk, dh, dv = self.hq, self.hkv, self.tq, self.tk, self.dh, self.dv
        rec = (lambda i: self.hip.hipEventRecord(events[i], sh)) if events is not None else (lambda i: 0)
        rec(0)
        st = L.rmm_qk(self.Qs[c].data_ptr(), self.Ks[c].data_ptr(), rmm.RMM_BF16, hq, hkv, tq, tk, dh, tq * dh, dh,
                      tk * dh, dh, float(rho), self.iq[rho].data_ptr(), self.S.data_ptr(), rmm.RMM_FP32,
                      self.wsq.data_ptr(), self.wsq.numel(), sh)
        if st != 0:
            raise RuntimeError(f"rmm_qk: {rmm.status_str(st)}")
        rec(1)
        if rho < 1.0:
            st = L.rmm_softmax_select(self.S.data_ptr(), float(dh) ** -0.5, hq, tq, tk, tq * tk, tk,
                                      self.P.data_ptr(), tq * tk, tk, self.E.data_ptr(), float(rho),
                                      self.ip[rho].data_ptr(), self.wss.data_ptr(), self.wss.numel(), sh)
            if st != 0:
                raise RuntimeError(f"rmm_softmax_select: {rmm.status_str(st)}")
            rec(2)
            rec(3)
            st = L.rmm_pv_idx(self.P.data_ptr(), rmm.RMM_FP32, self.Vs[c].data_ptr(), rmm.RMM_BF16,
                              self.ip[rho].data_ptr(), self.ks[rho], hq, hkv, tq, tk, dv, tq * tk, tk, tk * dv, dv,
                              self.O.data_ptr(), rmm.RMM_FP32, self.wsp.data_ptr(), self.wsp.numel(), sh)
            if st != 0:
                raise RuntimeError(f"rmm_pv_idx: {rmm.status_str(st)}")
        else:
            st = L.rmm_softmax_energy(self.S.data_ptr(), float(dh) ** -0.5, hq, tq, tk, tq * tk, tk,
                                      self.P.data_ptr(), tq * tk, tk, self.E.data_ptr(), self.wss.data_ptr(),
                                      self.wss.numel(), sh)
            if st != 0:
                raise RuntimeError(f"rmm_softmax_energy: {rmm.status_str(st)}")
            rec(2)
            rec(3)
            st = L.rmm_pv_energy(self.P.data_ptr(), rmm.RMM_FP32, self.Vs[c].data_ptr(), rmm.RMM_BF16,
                                 self.E.data_ptr(), hq, hkv, tq, tk, dv, tq * tk, tk, tk * dv, dv, float(rho),
                                 self.ip[rho].data_ptr(), self.O.data_ptr(), rmm.RMM_FP32, self.wsp.data_ptr(),
                                 self.wsp.numel(), sh)
            if st != 0:
                raise RuntimeError(f"rmm_pv_energy: {rmm.status_str(st)}")
        rec(4)

    def stage_work(self, rho):
        hq, hkv, tq, tk, dh, dv = self.hq, self.hkv, self.tq, self.tk, self.dh, self.dv
        s_bytes = hq * tq * tk * 4
        return {"qk": ("B", hkv * tk * dh * 2 + s_bytes),           # the key cache once per kv head, S
                "softmax": ("B", 2 * s_bytes),
                "pv": ("B", hq * self.ks[rho] * dv * 2 + s_bytes)}   # kept V rows per head, P

    def roofline_stage(self):
        return None

    def roofline_kernel(self):
        return {"qk": "qk_decode_kernel (streaming pass over the key cache)",
                "softmax": "softmax_select_kernel (softmax, key energies and the kept lists; dense: "
                           "softmax_energy_kernel)",
                "pv": "the rmm_pv_idx call: gemv_kernel batched over heads (the listed V rows) and "
                      "gemv_reduce_kernel (dense: rmm_pv_energy over every row)"}

    def traffic_ref(self):
        return None

    def shape(self):
        return {"shape": self.desc}

    def cpu_baseline(self):
        import numpy as np
        from oracle import rmm_oracle as O
        Q = self.Qs[0].float().cpu().numpy()
        K = self.Ks[0].float().cpu().numpy()
        V = self.Vs[0].float().cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while True:
            for rho in self.rhos:
                _, S = O.qk(Q, K, rho)
                P = O.softmax_rows(S, self.dh ** -0.5)
                E = np.stack([O.col_energy(P[h]) for h in range(self.hq)])
                O.pv_given_energy(P, V, E, rho)
            reps += 1
            if time.perf_counter() - t0 > CPU_SAMPLE_SECONDS:
                break
        wall = time.perf_counter() - t0
        return {"value": reps * len(self.rhos) / wall, "unit": "decode attention steps/s", "cores": _blas_threads(),
                "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(), "kind": "oracle",
                "sample": (f"fp64 oracle qk, row softmax, energies and pv on the whole step at each rho in "
                           f"{list(self.rhos)}, {reps} repetitions; {wall:.1f} s of CPU work")}


WORKLOADS = ("mlp_down_8b", "mlp_up_70b", "decode_qkv_8b", "gqa_qk_8b", "attn_pv_70b", "decode_attn_8b",
             "decode_qkv_8b_w8", "mlp_down_8b_w8")


def make_op(name, copies, strict=False):
    import synth
    if name == "mlp_down_8b":
        w = synth.mlp_down(strict_adjacent=strict)
        return MatmulOp(name, w.tensors["A"], w.tensors["B"], (0.9, 0.7, 0.5, 1.0),
                        "A 4096x14336 bf16 (log-normal channel scale, 1% outlier channels x20) @ "
                        "B 14336x4096 bf16 -> Y fp32", copies)
    if name == "mlp_up_70b":
        w = synth.mlp_up(strict_adjacent=strict)
        return MatmulOp(name, w.tensors["A"], w.tensors["B"], (0.8, 1.0),
                        "A 2048x8192 bf16 @ B 8192x28672 bf16 -> Y fp32", copies)
    if name == "decode_qkv_8b":
        w = synth.decode_qkv(strict_adjacent=strict)
        return MatmulOp(name, w.tensors["A"], w.tensors["B"], (0.8, 1.0),
                        "A 8x4096 bf16 @ B 4096x6144 bf16 -> Y fp32 (decode GEMV over kept rows)", copies)
    if name == "decode_qkv_8b_w8":
        w = synth.w8_projection(strict_adjacent=strict)
        return MatmulW8Op(name, w.tensors["A"], w.tensors["Bq"], w.tensors["scale"], (0.8, 1.0),
                          "A 8x4096 bf16 @ Bq 4096x6144 int8 (fp32 scale per column) -> Y fp32 "
                          "(decode GEMV over kept int8 rows)", copies)
    if name == "mlp_down_8b_w8":
        w = synth.w8_projection(n=4096, d=14336, m=4096, rho=0.7, workload=1, name=name, strict_adjacent=strict)
        return MatmulW8Op(name, w.tensors["A"], w.tensors["Bq"], w.tensors["scale"], (0.7, 1.0),
                          "A 4096x14336 bf16 @ Bq 14336x4096 int8 (fp32 scale per column) -> Y fp32", copies)
    if name == "gqa_qk_8b":
        w = synth.gqa_qk()
        return QkOp(name, w.tensors["Q"], w.tensors["K"], (0.5, 1.0),
                    "Q (32,4096,128) bf16, K (8,4096,128) bf16 (GQA group 4) -> S (32,4096,4096) fp32", copies)
    if name == "decode_attn_8b":
        wq = synth.decode_attn_qk(hq=32, hkv=8, tq=1, tk=8192, dh=128)
        wp = synth.attn_pv(h=32, hkv=8, tq=1, tk=8192, dv=128, strict_adjacent=strict)
        return DecodeAttnOp(name, wq.tensors["Q"], wq.tensors["K"], wp.tensors["V"], (0.5, 1.0),
                            "one query per head, Q (32,1,128) bf16, K and V caches (8,8192,128) bf16 (GQA group 4); "
                            "rho keeps features in QK^T and keys in PV", copies, _hip())
    w = synth.attn_pv(with_logits=True, strict_adjacent=strict)
    return PvOp(name, w.tensors["P"], w.tensors["V"], (0.5, 1.0),
                "P (64,512,8192) fp32 row-softmax, V (8,8192,128) bf16 (GQA group 8) -> O (64,512,128) fp32",
                copies, L_cpu=w.tensors["L"])


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp_down_8b", choices=WORKLOADS)
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (default: enough to exceed the "
                                                          "256 MB Infinity Cache)")
    ap.add_argument("--stage-iters", type=int, default=10, help="calls per rho with stage events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the hipBLASLt context timing")
    ap.add_argument("--strict-adjacent", action="store_true",
                    help="space every neighbouring pair of sorted scores (the literal separation reading) instead "
                         "of the selection boundaries only; changes the values, not the work")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    copies = args.copies
    if copies <= 0:
        copies = {"gqa_qk_8b": 8, "attn_pv_70b": 2, "decode_attn_8b": 8}.get(args.workload, 4)
    op = make_op(args.workload, copies, strict=args.strict_adjacent)
    line = run(args, op)
    line["hipblaslt_dense_bf16out_us_context"] = None if args.no_context else hipblaslt_context(op)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = op.cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
