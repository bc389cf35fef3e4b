"""Helpers that turn rocprofv3 output into the short summaries kept with the
library, and the copy kernel that calibrates the HBM byte counters.

    python -m input_adaptive_reduced_colnorm_amd.profiling copy --mib 256 --iters 3
        device-to-device copies of a known size (run under rocprofv3 --pmc to
        read what FETCH_SIZE / WRITE_SIZE report for a known byte count)
    python -m input_adaptive_reduced_colnorm_amd.profiling summarize STATS.csv OUT.md --title T --command C
        kernel statistics table (rocprofv3 --kernel-trace --stats)
    python -m input_adaptive_reduced_colnorm_amd.profiling traffic --fetch F.csv --write W.csv \\
            --copy-fetch CF.csv --copy-write CW.csv --copy-mib 256 --kernel SUBSTR \\
            --source FILE --workload NAME --out OUT.json
        HBM bytes per launch of one kernel from two counter runs, each scaled by
        what the same counter reads for the calibration copy

    python -m input_adaptive_reduced_colnorm_amd.profiling mfma --counters C.csv --kernel SUBSTR \
            --title T --command CMD --out OUT.md
        per launch of one kernel: shader clock (GRBM_GUI_ACTIVE of one XCD over
        the launch time), matrix-core busy share (SQ_VALU_MFMA_BUSY_CYCLES over
        the cycles of all 1024 SIMDs) and the bf16 MFMA rate from
        SQ_INSTS_VALU_MFMA_MOPS_BF16 (512 FLOP per count)

Nothing here is on the compute path; the JSON written by `traffic` records a
hash of the kernel source so that a reader can tell when it is stale.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _short_name(name: str) -> str:
    n = name.replace("rmm::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0] if "<" not in n else n[: n.index(">") + 1]


def summarize(stats_csv: str, out_md: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (from the repository root on one MI355X, TMPDIR=/tmp):", "", "```", command,
           "```", "", "Kernel statistics from `rocprofv3 --kernel-trace --stats` (durations in microseconds):", "",
           "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    text = "\n".join(out) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


def _counter_per_dispatch(path: str, counter: str, substr: str):
    """Counter value (summed over its instances) per dispatch of kernels whose
    name contains `substr`."""
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or substr not in r["Kernel_Name"]:
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(per.values())


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib, kernel, source, workload, out_json,
            copy_kernel="opy"):
    copy_bytes = copy_mib * (1 << 20)
    cf = _counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", copy_kernel)
    cw = _counter_per_dispatch(copy_write_csv, "WRITE_SIZE", copy_kernel)
    if not cf or not cw:
        raise SystemExit("no copy-kernel dispatches in the calibration runs")
    # counters are in KiB per dispatch
    fetch_factor = copy_bytes / (statistics.median(cf) * 1024.0)
    write_factor = copy_bytes / (statistics.median(cw) * 1024.0)
    f = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel)
    w = _counter_per_dispatch(write_csv, "WRITE_SIZE", kernel)
    if not f or not w:
        raise SystemExit(f"no dispatches of {kernel!r} in the counter runs")
    fetch_b = statistics.fmean(f) * 1024.0 * fetch_factor
    write_b = statistics.fmean(w) * 1024.0 * write_factor
    rec = {
        "kernel": kernel,
        "workload": workload,
        "kernel_source": os.path.relpath(source),
        "kernel_source_sha256": source_hash(source),
        "dispatches": {"fetch": len(f), "write": len(w)},
        "fetch_kib_per_dispatch_raw": round(statistics.fmean(f), 1),
        "write_kib_per_dispatch_raw": round(statistics.fmean(w), 1),
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib_raw": statistics.median(cf),
                             "write_kib_raw": statistics.median(cw), "fetch_factor": round(fetch_factor, 4),
                             "write_factor": round(write_factor, 4)},
        "hbm_bytes_per_launch": {"fetch": round(fetch_b), "write": round(write_b), "total": round(fetch_b + write_b)},
    }
    with open(out_json, "w") as fo:
        json.dump(rec, fo, indent=1)
        fo.write("\n")
    return rec


XCDS, SIMDS = 8, 1024           # MI355X: 8 accelerator complexes, 256 CUs x 4 SIMDs


def _dispatch_rows(path: str, substr: str):
    """{dispatch id: {"name", "ns", counter: summed value}} for kernels whose
    name contains `substr`."""
    out = {}
    for r in csv.DictReader(open(path)):
        if substr not in r["Kernel_Name"]:
            continue
        d = out.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                              "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def mfma(counters_csv: str, kernel: str, title: str, command: str, out_md: str) -> str:
    rows = _dispatch_rows(counters_csv, kernel)
    need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    rows = {k: v for k, v in rows.items() if all(c in v for c in need)}
    if not rows:
        raise SystemExit(f"no dispatches of {kernel!r} with {need}")
    out = [f"# {title}", "", "Command (from the repository root on one MI355X, TMPDIR=/tmp):", "", "```", command,
           "```", "", f"Kernel `{_short_name(next(iter(rows.values()))['name'])}`, one line per launch. Clock = "
           "GRBM_GUI_ACTIVE / 8 XCDs / launch time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 "
           "x 1024 SIMDs); TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / launch time; the last column scales "
           "the 2.5 PFLOP/s bf16 peak (quoted at 2.4 GHz) to the measured clock.", "",
           "| launch | us | clock GHz | MFMA busy | TFLOP/s | peak at that clock |", "|---|---|---|---|---|---|"]
    clocks, busy, tf = [], [], []
    for i, (k, v) in enumerate(sorted(rows.items(), key=lambda kv: int(kv[0]))):
        us = v["ns"] / 1e3
        cyc = v["GRBM_GUI_ACTIVE"] / XCDS
        ghz = cyc / (us * 1e3)
        b = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
        t = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (us * 1e-6) / 1e12
        clocks.append(ghz), busy.append(b), tf.append(t)
        out.append(f"| {i} | {us:.1f} | {ghz:.2f} | {b:.1%} | {t:.0f} | {2500 * ghz / 2.4:.0f} |")
    out += ["", f"Mean over {len(rows)} launches: clock {statistics.fmean(clocks):.2f} GHz, MFMA busy "
            f"{statistics.fmean(busy):.1%}, {statistics.fmean(tf):.0f} TFLOP/s."]
    text = "\n".join(out) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


def copy(mib: int, iters: int):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {iters}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=256)
    c.add_argument("--iters", type=int, default=3)
    s = sub.add_parser("summarize")
    s.add_argument("stats_csv")
    s.add_argument("out_md")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    for name in ("fetch", "write", "copy-fetch", "copy-write", "kernel", "source", "workload", "out"):
        t.add_argument("--" + name, required=True)
    t.add_argument("--copy-mib", type=int, default=256)
    t.add_argument("--copy-kernel", default="opy", help="name substring of the calibration copy kernel")
    m = sub.add_parser("mfma")
    for name in ("counters", "kernel", "title", "command", "out"):
        m.add_argument("--" + name, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        copy(a.mib, a.iters)
    elif a.cmd == "summarize":
        sys.stdout.write(summarize(a.stats_csv, a.out_md, a.title, a.command))
    elif a.cmd == "mfma":
        sys.stdout.write(mfma(a.counters, a.kernel, a.title, a.command, a.out))
    else:
        print(json.dumps(traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.kernel, a.source,
                                 a.workload, a.out, a.copy_kernel), indent=1))


if __name__ == "__main__":
    main()
