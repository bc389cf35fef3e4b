#!/usr/bin/env python3
"""Benchmark of the RMM hot path on one MI355X.

Default workload: the Llama-3.1-8B MLP down projection in prefill,
A 4096 x 14336 bf16 activations times B 14336 x 4096 bf16 weights, fp32 Y.
One step = one rmm_matmul call at each retention ratio 0.9, 0.7 and 0.5
(score, TopK, gather-pack, reduced GEMM) plus the rho = 1 dense product
that the speedups are measured against.  Inputs are resident in HBM before
the timed region; four copies of (A, B) are rotated so that consecutive
calls do not find their operands in the 256 MB Infinity Cache.

Per-kernel times come from HIP events that the library records on its own
stream at the stage boundaries (rmm_matmul_timed).  Prints ONE JSON line.

Other workloads (--workload) print the same kind of line for profiling; the
driver uses the default.
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


def _die_multi_gpu(n):
    print(json.dumps({"error": f"--gpus {n}: this build measures one GPU only; the path has no multi-GPU "
                               "collective (see DESIGN.md for how it would shard)"}))
    sys.exit(2)


def _hip():
    import torch  # noqa: F401  (loads the HIP runtime librmm shares)
    lib_dir = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    h = ctypes.CDLL(lib_dir if os.path.exists(lib_dir) else "libamdhip64.so.7")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
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


def cpu_baseline_matmul(A_cpu, B_cpu, rhos, sample_rows):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from oracle import rmm_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = sum(int(p.get("num_threads", 1)) for p in threadpool_info() if p.get("user_api") == "blas")
    except Exception:  # pragma: no cover - informational only
        threads = os.cpu_count()
    A = A_cpu.float().numpy()
    B = B_cpu.float().numpy()
    n = A.shape[0]
    rows = np.arange(sample_rows)
    est = {}
    wall = 0.0
    for rho in rhos:
        t0 = time.perf_counter()
        O.select(A, rho)
        t1 = time.perf_counter()
        O.matmul(A, B, rho, rows=rows)
        t2 = time.perf_counter()
        t_sel = t1 - t0
        t_prod = max(t2 - t1 - t_sel, 0.0)
        est[rho] = t_sel + t_prod * n / sample_rows
        wall += t2 - t0
    total = sum(est.values())
    return {
        "value": len(rhos) / total,
        "unit": "RMM ops/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"full fp64 scoring + stable-sort TopK on all {n} rows, reduced product on rows 0..{sample_rows - 1} "
                   f"of {n}, scaled by {n // sample_rows}x; one call per rho in {list(rhos)}; "
                   f"{wall:.1f} s of CPU work"),
        "est_op_s": {str(r): round(v, 4) for r, v in est.items()},
    }


def bench_matmul(args, name, A_cpu, B_cpu, rhos, desc):
    import torch
    from input_adaptive_reduced_colnorm_amd import rmm

    dev = torch.device("cuda:0")
    hip = _hip()
    L = rmm.lib()
    n, d = A_cpu.shape
    m = B_cpu.shape[1]
    copies = max(1, args.copies)
    As = [A_cpu.to(dev) for _ in range(copies)]
    Bs = [B_cpu.to(dev) for _ in range(copies)]
    Y = torch.empty((n, m), dtype=torch.float32, device=dev)
    ks = {r: rmm.k(r, d) for r in rhos}
    idx = {r: torch.empty(ks[r], dtype=torch.int32, device=dev) for r in rhos}
    ws_bytes = max(int(L.rmm_matmul_workspace(n, d, m, d, rmm.RMM_BF16, r)) for r in rhos)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    nops = len(rhos)
    evs = Events(hip, 5 * args.stage_iters * nops)

    def call_timed(c, rho, slot):
        st = L.rmm_matmul_timed(As[c].data_ptr(), Bs[c].data_ptr(), rmm.RMM_BF16, n, d, m, d, m, float(rho),
                                idx[rho].data_ptr(), Y.data_ptr(), rmm.RMM_FP32, m, ws.data_ptr(), ws.numel(), sh,
                                evs.array(5 * slot))
        if st != 0:
            raise RuntimeError(f"rmm_matmul_timed: {rmm.status_str(st)}")

    def call(c, rho):
        st = L.rmm_matmul(As[c].data_ptr(), Bs[c].data_ptr(), rmm.RMM_BF16, n, d, m, d, m, float(rho),
                          idx[rho].data_ptr(), Y.data_ptr(), rmm.RMM_FP32, m, ws.data_ptr(), ws.numel(), sh)
        if st != 0:
            raise RuntimeError(f"rmm_matmul: {rmm.status_str(st)}")

    for step in range(args.warmup):
        for j, rho in enumerate(rhos):
            call((step * nops + j) % copies, rho)
    torch.cuda.synchronize()

    # timed region: K steps; barrier (single process) + device sync on both sides
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for step in range(args.steps):
        for j, rho in enumerate(rhos):
            call((step * nops + j) % copies, rho)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # op latency per rho: back-to-back calls between two events (no events
    # between calls: an event record costs a few microseconds of GPU time)
    op_us = {}
    for j, rho in enumerate(rhos):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for it in range(args.steps):
            call((it + j) % copies, rho)
        e1.record(stream)
        torch.cuda.synchronize()
        op_us[rho] = e0.elapsed_time(e1) / args.steps * 1e3

    # per-kernel durations: the same calls with stage events recorded by the
    # library on its stream (rmm_matmul_timed)
    stages = {r: {"score": [], "topk": [], "pack": [], "gemm": [], "op": []} for r in rhos}
    slot = 0
    for it in range(args.stage_iters):
        for j, rho in enumerate(rhos):
            call_timed((it * nops + j) % copies, rho, slot)
            slot += 1
    torch.cuda.synchronize()
    slot = 0
    for it in range(args.stage_iters):
        for rho in rhos:
            b = 5 * slot
            st = stages[rho]
            st["score"].append(evs.ms(b, b + 1))
            st["topk"].append(evs.ms(b + 1, b + 2))
            st["pack"].append(evs.ms(b + 2, b + 3))
            st["gemm"].append(evs.ms(b + 3, b + 4))
            st["op"].append(evs.ms(b, b + 4))
            slot += 1
    evs.close()

    med = {r: {k2: statistics.median(v) * 1e3 for k2, v in stages[r].items()} for r in rhos}  # us
    mean = {r: {k2: statistics.fmean(v) * 1e3 for k2, v in stages[r].items()} for r in rhos}
    dense_r = 1.0 if 1.0 in rhos else None
    lat = {str(r): round(op_us[r], 2) for r in rhos}
    speed = {}
    if dense_r is not None:
        for r in rhos:
            if r != dense_r:
                speed[str(r)] = round(op_us[dense_r] / op_us[r], 4)

    def gemm_flops(r):
        return 2.0 * n * ks[r] * m

    per_kernel = {}
    for r in rhos:
        e = mean[r]
        row = {
            "gemm_us": round(e["gemm"], 2),
            "gemm_tflops": round(gemm_flops(r) / (e["gemm"] * 1e-6) / 1e12, 1),
            "gemm_mfma_frac": round(gemm_flops(r) / (e["gemm"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
        }
        if r != dense_r:
            a_bytes = n * d * 2
            row["score_us"] = round(e["score"], 2)
            row["score_gbs"] = round(a_bytes / (e["score"] * 1e-6) / 1e9, 1)
            row["score_hbm_frac"] = round(a_bytes / (e["score"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            row["topk_us"] = round(e["topk"], 2)
            pk_bytes = 2 * n * ks[r] * 2
            row["pack_us"] = round(e["pack"], 2)
            row["pack_gbs"] = round(pk_bytes / (e["pack"] * 1e-6) / 1e9, 1)
            row["pack_hbm_frac"] = round(pk_bytes / (e["pack"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        per_kernel[str(r)] = row

    # dominant kernel: the reduced product kernel, averaged over its launches (rho < 1)
    red = [r for r in rhos if r != dense_r]
    tot_s = sum(mean[r]["gemm"] * 1e-6 for r in red)
    if n <= 16:
        # decode: the GEMV streams the kept rows of B (k x m bf16)
        for r in rhos:
            per_kernel[str(r)]["gemv_gbs"] = round(ks[r] * m * 2 / (mean[r]["gemm"] * 1e-6) / 1e9, 1)
            per_kernel[str(r)]["gemv_hbm_frac"] = round(ks[r] * m * 2 / (mean[r]["gemm"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        tot_b = sum(ks[r] * m * 2 for r in red)
        achieved = tot_b / tot_s / 1e9
        roofline = {
            "kernel": "gemv_kernel (kept rows of B, mean over rho in %s)" % red,
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
            "per_launch_bytes": {str(r): ks[r] * m * 2 for r in red},
            "avg_launch_us": round(tot_s / len(red) * 1e6, 2),
        }
    else:
        tot_flops = sum(gemm_flops(r) for r in red)
        achieved = tot_flops / tot_s / 1e12
        roofline = {
            "kernel": "gemm_bf16_kernel<256,256,kmajor,gather> (reduced GEMM, mean over rho in %s)" % red,
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "per_launch_flops": {str(r): gemm_flops(r) for r in red},
            "avg_launch_us": round(tot_s / len(red) * 1e6, 2),
        }

    # hipBLASLt dense time at the same shape, as context only (bf16 output)
    ctx = None
    if not args.no_context:
        Ad, Bd = As[0], Bs[0]
        for _ in range(3):
            torch.matmul(Ad, Bd)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(Ad, Bd)
        e1.record()
        torch.cuda.synchronize()
        ctx = round(e0.elapsed_time(e1) / 10 * 1e3, 1)

    line = {
        "metric": METRIC,
        "value": round(nops * args.steps / (ms_total * 1e-3), 2),
        "unit": "RMM ops/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "shape": desc, "rhos": list(rhos),
                   "k": {str(r): ks[r] for r in rhos}, "copies_rotated": copies},
        "latency_us": lat,
        "latency_note": "per-op mean of back-to-back rmm_matmul calls; kernel times below come from stage events",
        "speedup_vs_dense": speed,
        "kernels": per_kernel,
        "roofline": roofline,
        "hipblaslt_dense_bf16out_us_context": ctx,
    }
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp_down_8b", choices=["mlp_down_8b", "mlp_up_70b", "decode_qkv_8b"])
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--stage-iters", type=int, default=10, help="calls per rho with stage events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the hipBLASLt context timing")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth

    if args.workload == "mlp_down_8b":
        w = synth.mlp_down()
        rhos = (0.9, 0.7, 0.5, 1.0)
        desc = "A 4096x14336 bf16 (log-normal channel scale, 1% outlier channels x20) @ B 14336x4096 bf16 -> Y fp32"
    elif args.workload == "mlp_up_70b":
        w = synth.mlp_up()
        rhos = (0.8, 1.0)
        desc = "A 2048x8192 bf16 @ B 8192x28672 bf16 -> Y fp32"
    else:
        w = synth.decode_qkv()
        rhos = (0.8, 1.0)
        desc = "A 8x4096 bf16 @ B 4096x6144 bf16 -> Y fp32 (decode GEMV over kept rows)"
    A_cpu, B_cpu = w.tensors["A"], w.tensors["B"]
    line = bench_matmul(args, args.workload, A_cpu, B_cpu, rhos, desc)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_matmul(A_cpu, B_cpu, rhos, sample_rows=min(1024, A_cpu.shape[0]))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
