"""Summaries of rocprofv3 output for the measurement notes (kernel-trace statistics and
per-dispatch HBM counters). Reads the CSV files rocprofv3 writes with --output-format csv;
runs no GPU code."""
from __future__ import annotations

import csv
import glob
import os
import sys
from collections import defaultdict


def _rows(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def kernel_stats(d: str) -> list[tuple[str, int, float, float, float]]:
    """(kernel, calls, avg_us, min_us, max_us) from the kernel trace, by total time."""
    acc = defaultdict(list)
    for r in _rows(d, "kernel_trace.csv"):
        acc[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    out = [(k, len(v), sum(v) / len(v), min(v), max(v)) for k, v in acc.items()]
    return sorted(out, key=lambda x: -x[1] * x[2])


def counter_means(d: str, counter: str) -> dict[str, tuple[int, float]]:
    """kernel -> (dispatches, mean counter value per dispatch)."""
    per = defaultdict(lambda: defaultdict(float))
    for r in _rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (len(v), sum(v.values()) / len(v)) for k, v in per.items()}


def per_dispatch(d: str, counter: str) -> list[tuple[int, str, float]]:
    """(dispatch id, kernel, counter value summed over its instances) for every dispatch."""
    per, names = defaultdict(float), {}
    for r in _rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        i = int(r["Dispatch_Id"])
        per[i] += float(r["Counter_Value"])
        names[i] = r["Kernel_Name"]
    return [(i, names[i], v) for i, v in sorted(per.items())]


def dispatch_ns(d: str) -> dict[int, float]:
    """dispatch id -> its duration in ns, from the start / end timestamps of the counter rows."""
    out = {}
    for r in _rows(d, "counter_collection.csv"):
        out[int(r["Dispatch_Id"])] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def mfma(d: str, simds: int = 1024, clock_ghz: float = 2.4) -> list[dict]:
    """Per kernel, from one run with SQ_INSTS_VALU_MFMA_MOPS_BF16 and SQ_VALU_MFMA_BUSY_CYCLES:
    bf16 MFMA flops per dispatch (MOPS x 512), the flop rate over the dispatch's own duration
    (its timestamps), and the MFMA busy share of the SIMDs (busy cycles summed over the SIMDs /
    (duration x clock_ghz x simds)). GRBM_GUI_ACTIVE is not used as the denominator: in a
    counter run it also counts cycles outside the dispatch."""
    mops = {i: (k, v) for i, k, v in per_dispatch(d, "SQ_INSTS_VALU_MFMA_MOPS_BF16")}
    busy = {i: v for i, _, v in per_dispatch(d, "SQ_VALU_MFMA_BUSY_CYCLES")}
    dur = dispatch_ns(d)
    acc = defaultdict(lambda: [0, 0.0, 0.0, 0.0])
    for i, (k, m) in mops.items():
        if i not in busy or dur.get(i, 0.0) <= 0:
            continue
        a = acc[k]
        a[0] += 1
        a[1] += 512.0 * m
        a[2] += busy[i]
        a[3] += dur[i]
    out = []
    for k, (n, fl, bu, ns) in acc.items():
        t = ns / n * 1e-9
        out.append({"kernel": k, "dispatches": n, "flops_per_dispatch": fl / n, "duration_us": t * 1e6,
                    "tflops": fl / n / t / 1e12, "mfma_busy_pct": 100.0 * bu / (ns * clock_ghz * simds)})
    return sorted(out, key=lambda r: -r["flops_per_dispatch"] * r["dispatches"])


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int) -> dict:
    """HBM bytes per dispatch of `kernel` from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by copy_bytes over what the counter reads for the plain device copy of
    copy_bytes (the copy dispatches are those reading / writing at least half of it)."""
    out = {}
    for d, c in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = per_dispatch(d, c)
        copies = [v for _, k, v in rows if "copyBuffer" in k and v * 1024 >= copy_bytes / 4]
        mine = [v for _, k, v in rows if kernel in k]
        if not copies or not mine:
            raise ValueError(f"{c}: copy or kernel dispatches not found")
        scale = copy_bytes / (1024 * sum(copies) / len(copies))
        out[c] = {"kib_per_dispatch": sum(mine) / len(mine), "dispatches": len(mine), "copy_kib": sum(copies) / len(copies),
                  "scale": scale, "bytes_per_dispatch": scale * 1024 * sum(mine) / len(mine)}
    out["bytes_per_dispatch"] = out["FETCH_SIZE"]["bytes_per_dispatch"] + out["WRITE_SIZE"]["bytes_per_dispatch"]
    return out


def source_hash(files: list[str]) -> str:
    """sha256 over the given source files, to tie counter figures to one kernel version."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


LOOP_SOURCES = ["csrc/fm_xloop.hip", "csrc/fm_xloop.h", "csrc/fm_common.h"]
GRAPH_SOURCES = ["csrc/fm_gemm.hip", "csrc/fm_attn.hip", "csrc/fm_kernels.h", "csrc/fm_common.h"]


def loop_source_hash() -> str:
    here = os.path.dirname(os.path.abspath(__file__))
    return source_hash([os.path.join(here, f) for f in LOOP_SOURCES])


def graph_source_hash() -> str:
    """sha256 of the per-operation kernels' sources (the GEMMs and the attention)."""
    here = os.path.dirname(os.path.abspath(__file__))
    return source_hash([os.path.join(here, f) for f in GRAPH_SOURCES])


def main(argv):
    """profiling.py stats DIR | counters DIR COUNTER | mfma DIR | traffic FETCH_DIR WRITE_DIR KERNEL COPY_BYTES"""
    if argv[0] == "stats":
        rows = kernel_stats(argv[1])
        tot = sum(c * a for _, c, a, _, _ in rows)
        print(f"# total kernel time {tot / 1000:.3f} ms")
        print(f"{'kernel':80s} {'calls':>7s} {'avg_us':>10s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}")
        for k, c, a, lo, hi in rows:
            print(f"{k[:80]:80s} {c:7d} {a:10.2f} {lo:9.2f} {hi:9.2f} {100 * c * a / tot:7.2f}")
    elif argv[0] == "counters":
        for k, (n, m) in sorted(counter_means(argv[1], argv[2]).items(), key=lambda x: -x[1][1]):
            print(f"{argv[2]} {m:14.1f} KiB/dispatch x{n:3d}  {k[:100]}")
    elif argv[0] == "mfma":
        rows = mfma(argv[1])
        print(f"{'kernel':80s} {'disp':>5s} {'GFLOP/disp':>11s} {'us/disp':>9s} {'TFLOP/s':>8s} {'%2.5PF':>7s} {'busy%':>6s}")
        for r in rows:
            print(f"{r['kernel'][:80]:80s} {r['dispatches']:5d} {r['flops_per_dispatch'] / 1e9:11.3f} "
                  f"{r['duration_us']:9.2f} {r['tflops']:8.1f} {100 * r['tflops'] / 2500:7.2f} {r['mfma_busy_pct']:6.1f}")
        mm = [r for r in rows if r["flops_per_dispatch"] > 0]
        tt = sum(r["duration_us"] * r["dispatches"] for r in mm)
        print(f"mfma_busy_pct_time_weighted: {sum(r['mfma_busy_pct'] * r['duration_us'] * r['dispatches'] for r in mm) / tt:.2f}")
        print(f"source_sha256: {graph_source_hash()}")
    elif argv[0] == "traffic":
        t = traffic(argv[1], argv[2], argv[3], int(argv[4]))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            x = t[c]
            print(f"{c}: {x['kib_per_dispatch']:.1f} KiB per dispatch over {x['dispatches']} dispatches; "
                  f"plain copy of {int(argv[4])} bytes reads {x['copy_kib']:.1f} KiB -> scale {x['scale']:.4f}; "
                  f"{x['bytes_per_dispatch']:.0f} bytes per dispatch")
        print(f"traffic_bytes_per_launch: {t['bytes_per_dispatch']:.0f}")
        print(f"source_sha256: {loop_source_hash()}")
    else:
        raise SystemExit(main.__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
