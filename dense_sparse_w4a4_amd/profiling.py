"""Summaries of rocprofv3 output for the fused-layer kernels.

    python -m dense_sparse_w4a4_amd.profiling stats  OUTDIR PREFIX TITLE CMD > summary.md
    python -m dense_sparse_w4a4_amd.profiling traffic FETCH_DIR WRITE_DIR WORKLOAD KERNEL CMD > traffic.json

`stats` turns a `rocprofv3 --kernel-trace --stats -f csv` output directory
into a short markdown table (per kernel, and per launch shape of the fused
GEMM kernels).  `traffic` combines two `rocprofv3 --pmc FETCH_SIZE` /
`--pmc WRITE_SIZE` runs of `bench.py --copy-calibration` into HBM bytes per
fused-GEMM launch: each counter is scaled by the ratio of the known bytes of
the plain device copy in the same run (256 MiB read, 256 MiB written) to
what the same counter reports for that copy.  The result carries a hash of
the kernel sources; bench.py reports it only while the sources match.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20
COPY_KERNEL = "copyBuffer"


# the sources a fused-GEMM kernel's code and launch configuration come from
KERNEL_SOURCES = {
    "gemm_stream_kernel": ["gemm.hip"],
    "gemm_tile_kernel": ["gemm_tile.hip"],
    "gemm_tile6_kernel": ["gemm_tile6.hip", "fp6.hip"],
}
SHARED_SOURCES = ["api.hip", "gemm_common.h", "mq_internal.h"]


def kernel_sources_sha(kernel: str | None = None) -> str:
    """Hash of the sources `kernel` is built and launched from (every file
    under csrc/ when the kernel is not one of the fused-GEMM kernels)."""
    csrc = os.path.join(PKG, "csrc")
    if kernel in KERNEL_SOURCES:
        files = sorted(KERNEL_SOURCES[kernel] + SHARED_SOURCES)
    else:
        files = sorted(os.listdir(csrc))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _stamp(kernel: str | None = None) -> str:
    """Where a summary comes from: the commit named by MQ_COMMIT (the GPU
    host has the tree, not the history) and the kernel sources' hash."""
    c = os.environ.get("MQ_COMMIT", "unrecorded")
    return f"Taken on commit {c}; kernel sources sha {kernel_sources_sha(kernel)}."


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def _short(name: str) -> str:
    name = name.replace("mq::(anonymous namespace)::", "").replace("(mq::GemmArgs)", "")
    return name[:90]


def _pct(v, q: float) -> float:
    """q-th percentile (linear interpolation between order statistics)."""
    v = sorted(v)
    if len(v) == 1:
        return v[0]
    x = (len(v) - 1) * q / 100.0
    i = int(x)
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (x - i)


def stats(outdir: str, prefix: str, title: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(outdir, f"{prefix}_kernel_stats.csv")))))
    trace = list(csv.DictReader(open(_one(os.path.join(outdir, f"{prefix}_kernel_trace.csv")))))
    out = [f"# {title}", "", _stamp(), "", "Command (from the repository root on the GPU host):", "", "```", cmd,
           "```", "", "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:12]:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    # fused GEMM launches by kernel and grid (the grid identifies the shape)
    per = defaultdict(list)
    for t in trace:
        if "gemm_" in t["Kernel_Name"]:
            key = (_short(t["Kernel_Name"]), int(t["Grid_Size_X"]), int(t["Workgroup_Size_X"]))
            per[key].append((int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) / 1e3)
    if per:
        out += ["", "Fused GEMM launches by grid:", "",
                "| kernel | grid (threads) | block | calls | average (us) | p10 / median / p90 (us) |",
                "|---|---:|---:|---:|---:|---:|"]
        for (k, g, b), v in sorted(per.items()):
            out.append(f"| `{k}` | {g} | {b} | {len(v)} | {sum(v) / len(v):.2f} | "
                       f"{_pct(v, 10):.2f} / {_pct(v, 50):.2f} / {_pct(v, 90):.2f} |")
        # every template instance of a kernel together (the figure the
        # benchmark's per-launch average compares with)
        fam = defaultdict(list)
        for (k, _, _), v in per.items():
            for name in ("gemm_stream_kernel", "gemm_tile_kernel", "gemm_tile6_kernel"):
                if name + "<" in k or k.startswith(name):
                    fam[name] += v
        out += ["", "All launches per kernel (every template instance):", "",
                "| kernel | calls | average (us) | p10 / median / p90 (us) |", "|---|---:|---:|---:|"]
        for name, v in sorted(fam.items()):
            out.append(f"| `{name}` | {len(v)} | {sum(v) / len(v):.2f} | "
                       f"{_pct(v, 10):.2f} / {_pct(v, 50):.2f} / {_pct(v, 90):.2f} |")
    return "\n".join(out) + "\n"


def _counter(path: str, counter: str):
    per_kernel = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per_kernel[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per_kernel


def traffic(fetch_dir: str, write_dir: str, workload: str, kernel: str, cmd: str) -> dict:
    fetch = _counter(_one(os.path.join(fetch_dir, "*counter_collection.csv")), "FETCH_SIZE")
    write = _counter(_one(os.path.join(write_dir, "*counter_collection.csv")), "WRITE_SIZE")

    def pick(d, sub):
        vals = [v for k, vs in d.items() if sub in k for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel containing '{sub}'")
        return vals

    # the calibration copy is the largest copyBuffer dispatch
    fc = max(pick(fetch, COPY_KERNEL))
    wc = max(pick(write, COPY_KERNEL))
    f_k = pick(fetch, kernel)
    w_k = pick(write, kernel)
    ff = COPY_BYTES / (fc * 1024.0)
    fw = COPY_BYTES / (wc * 1024.0)
    # the write counter reads a plain copy's bytes exactly on this part: any
    # other factor means the largest copy of the run was not the calibration copy
    if not 0.95 <= fw <= 1.05:
        raise SystemExit(f"calibration copy not found: WRITE_SIZE of the largest copy is {wc:.0f} KiB, "
                         f"expected {COPY_BYTES / 1024:.0f}")
    fetch_kib = sum(f_k) / len(f_k)
    write_kib = sum(w_k) / len(w_k)
    return {
        "workload": workload,
        "kernel": kernel,
        "sources_sha": kernel_sources_sha(kernel),
        "commit": os.environ.get("MQ_COMMIT", "unrecorded"),
        "dispatches": len(f_k),
        "fetch_kib_per_dispatch": round(fetch_kib, 1),
        "write_kib_per_dispatch": round(write_kib, 1),
        "copy_fetch_kib": fc,
        "copy_write_kib": wc,
        "fetch_scale": round(ff, 4),
        "write_scale": round(fw, 4),
        "bytes_per_launch": round((fetch_kib * ff + write_kib * fw) * 1024.0),
        "command": cmd,
    }


# MI355X: 256 compute units of 4 SIMDs, in 8 XCDs of 4 shader engines.
N_SIMD = 1024
N_SE = 32


def sq(dirs, workload: str, kernel: str, cmd: str) -> str:
    """Per-dispatch means of SQ counters for one kernel, with derived shares.

    SQ_BUSY_CYCLES is summed over shader engines (kernel cycles = value /
    N_SE); SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES over SIMDs
    (cycles); SQ_WAVE_CYCLES, SQ_WAIT_*, SQ_ACTIVE_INST_* over waves, in
    units of 4 cycles."""
    vals = defaultdict(list)
    clocks = []  # (SQ_BUSY_CYCLES / N_SE) / dispatch duration, GHz
    for d in dirs:
        for r in csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv")))):
            if kernel in r["Kernel_Name"]:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "SQ_BUSY_CYCLES":
                    ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                    if ns > 0:
                        clocks.append(float(r["Counter_Value"]) / N_SE / ns)
    if not vals:
        raise SystemExit(f"no dispatch of a kernel containing '{kernel}'")
    m = {k: sum(v) / len(v) for k, v in vals.items()}
    out = [f"# SQ counters, `{kernel}`, workload {workload}", "", _stamp(kernel), "",
           "Commands (from the repository root on the GPU host):", "",
           "```", cmd, "```", "",
           "| counter | mean per dispatch | dispatches |", "|---|---:|---:|"]
    for k in sorted(m):
        out.append(f"| {k} | {m[k]:.0f} | {len(vals[k])} |")
    out += ["", "Derived (MI355X: 1024 SIMDs, 32 shader engines):", ""]
    if "SQ_BUSY_CYCLES" in m:
        cyc = m["SQ_BUSY_CYCLES"] / N_SE
        out.append(f"- kernel cycles (SQ_BUSY_CYCLES / 32): {cyc:.0f}")
        if clocks:
            out.append(f"- observed shader clock (kernel cycles / dispatch duration): "
                       f"{_pct(clocks, 50):.2f} GHz median ({min(clocks):.2f}-{max(clocks):.2f})")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            out.append(f"- matrix-core busy share per SIMD: {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMD * cyc):.1%}")
        if "SQ_ACTIVE_INST_VALU" in m:
            out.append(f"- vector-unit issue share per SIMD (ACTIVE_INST_VALU x 4 cycles, MFMA issue included): "
                       f"{4 * m['SQ_ACTIVE_INST_VALU'] / (N_SIMD * cyc):.1%}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        out.append(f"- matrix-core busy cycles with vector work co-issued: "
                   f"{m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.1%}")
    if "SQ_WAVE_CYCLES" in m:
        w = m["SQ_WAVE_CYCLES"]
        for k, what in (("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_WAIT_ANY", "waiting on a counter (s_waitcnt)"),
                        ("SQ_WAIT_INST_ANY", "instruction ready but not issued")):
            if k in m:
                out.append(f"- wave time {what}: {m[k] / w:.1%}")
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 5 and argv[0] == "stats":
        sys.stdout.write(stats(argv[1], argv[2], argv[3], argv[4]))
    elif len(argv) >= 5 and argv[0] == "sq":
        sys.stdout.write(sq(argv[1:-3], argv[-3], argv[-2], argv[-1]))
    elif len(argv) >= 6 and argv[0] == "traffic":
        json.dump(traffic(argv[1], argv[2], argv[3], argv[4], argv[5]), sys.stdout, indent=1)
        sys.stdout.write("\n")
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
