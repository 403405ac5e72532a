"""Summaries of rocprofv3 output for the layer's kernels.

Two summaries, each a short text file that names the command it came from:

* ``stats``: the kernel-trace statistics (calls, average and total duration
  per kernel) of one run.
* ``counters``: mean per-dispatch values of the SQ/GRBM counters of one
  kernel over one or more counter runs, with the clock and the MFMA, VALU and
  LDS mix derived from them.
* ``traffic``: HBM bytes per launch of one kernel from two counter runs (one
  with FETCH_SIZE, one with WRITE_SIZE).  The counters read in KiB per
  dispatch and do not count every byte the fabric moves, so each is scaled by
  what the same counter reads for a plain device-to-device copy of known size
  in the same run (``bench.py --copy-calibration MIB`` adds such copies).

The traffic summary also records a digest of the kernel's source files; a
reader (``load_traffic``) returns nothing once those files have changed, so a
figure is never reported for a kernel it was not measured on.

Usage::

    python -m llama2_decoder_layer_amd.profiling stats RUN_kernel_stats.csv --cmd "..."
    python -m llama2_decoder_layer_amd.profiling traffic FETCH.csv WRITE.csv \\
        --kernel gemm_gate_up --workload prefill_13b_t4096 --copy-mib 1024 --cmd "..."
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(PKG, "csrc")

# Kernel instances behind each timed kernel id, as rocprofv3 names them, and
# the source files they are compiled from.
_COMMON = ["common.cuh", "epilogue.cuh", "kernels.h"]
KERNELS = {
    "gemv_gate_up": (r"gemv_\w+_kernel<\d+, 2,", ["gemv.hip", "gemv_dma.hip"] + _COMMON),
    "gemm_gate_up": (r"gemm_(dma_)?kernel<\d+, 2,", ["gemm.hip"] + _COMMON),
    "gemm_qkv": (r"gemm_(dma_)?kernel<\d+, 0,", ["gemm.hip"] + _COMMON),
    "attn_prefill": (r"attn_prefill(_tr)?_kernel<", ["attn_prefill.hip"] + _COMMON),
    "attn_decode": (r"attn_(split|gqa)_kernel<", ["attn_decode.hip"] + _COMMON),
    "sample": (r"sample_kernel<", ["sample.hip"] + _COMMON),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
NOTE = "(REPO is the repository root, OUT the output directory.)"


def sources_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNELS[kernel][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("ll::", "")
    return name.split("(")[0]


def kernel_stats(path: str) -> list[dict]:
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append({"name": _short(r["Name"]), "calls": int(r["Calls"]),
                     "avg_us": float(r["AverageNs"]) / 1e3, "total_ms": float(r["TotalDurationNs"]) / 1e6,
                     "pct": float(r["Percentage"])})
    return rows


def format_stats(rows: list[dict], cmd: str, title: str) -> str:
    out = [f"# {title}", "", "Command:", "", "    " + cmd, "", NOTE, "",
           "| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.2f} | {r['total_ms']:.3f} | "
                   f"{r['pct']:.1f} |")
    return "\n".join(out) + "\n"


def counter_means(path: str) -> dict:
    """{(kernel, counter): (mean value, dispatches)} over one counter run."""
    acc = collections.defaultdict(list)
    grid = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        k = _short(r["Kernel_Name"])
        acc[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
        grid[(k, r["Counter_Name"])].append(int(r["Grid_Size"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}, grid, acc


def _copy_reading(path: str, counter: str) -> float:
    """The counter's reading for the largest copy dispatch (the calibration copy)."""
    _, grid, acc = counter_means(path)
    key = (COPY_KERNEL, counter)
    if key not in acc:
        raise SystemExit(f"{path}: no {COPY_KERNEL} dispatches (run bench.py with --copy-calibration)")
    g = grid[key]
    big = max(g)
    vals = [v for v, gs in zip(acc[key], g) if gs == big]
    return sum(vals) / len(vals)


def _kernel_reading(path: str, counter: str, kernel: str) -> tuple[float, int, str]:
    means, _, _ = counter_means(path)
    pat = re.compile(KERNELS[kernel][0])
    hits = [(k[0], v) for k, v in means.items() if k[1] == counter and pat.search(k[0])]
    if len(hits) != 1:
        raise SystemExit(f"{path}: {len(hits)} kernels match {kernel}: {[h[0] for h in hits]}")
    name, (val, n) = hits[0]
    return val, n, name


def traffic_summary(fetch_csv: str, write_csv: str, kernel: str, workload: str, copy_mib: float,
                    cmd_fetch: str, cmd_write: str) -> str:
    copy_bytes = copy_mib * 2**20
    f_copy = _copy_reading(fetch_csv, "FETCH_SIZE")
    w_copy = _copy_reading(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (f_copy * 1024)
    w_scale = copy_bytes / (w_copy * 1024)
    f_kib, nf, name = _kernel_reading(fetch_csv, "FETCH_SIZE", kernel)
    w_kib, nw, _ = _kernel_reading(write_csv, "WRITE_SIZE", kernel)
    fetch_b = f_kib * 1024 * f_scale
    write_b = w_kib * 1024 * w_scale
    lines = [
        f"# HBM traffic of {kernel} (`{name}`), workload {workload}",
        "",
        "FETCH_SIZE command:", "", "    " + cmd_fetch, "",
        "WRITE_SIZE command:", "", "    " + cmd_write, "",
        NOTE, "",
        f"Calibration: a device-to-device copy of {copy_mib:g} MiB reads FETCH_SIZE {f_copy:.0f} KiB "
        f"and WRITE_SIZE {w_copy:.0f} KiB per dispatch, so FETCH_SIZE is scaled by {f_scale:.3f} "
        f"and WRITE_SIZE by {w_scale:.3f}.",
        "",
        f"kernel: {name}",
        f"dispatches: fetch {nf}, write {nw}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"sources_sha256: {sources_digest(kernel)}",
    ]
    return "\n".join(lines) + "\n"


def counters_summary(csv_paths: list, kernel: str, workload: str, cmds: list) -> str:
    """Mean per-dispatch value of every counter collected for `kernel` over
    one or more counter runs (one file per run), with derived ratios: the
    shader clock (GRBM_GUI_ACTIVE counts GPU-active cycles summed over the 8
    XCDs, divided by the dispatch's duration in the same run), MFMA busy per
    busy CU cycle, and the VALU and LDS instruction mix per MFMA."""
    pat = re.compile(KERNELS[kernel][0])
    vals, names, dur = {}, set(), {}
    for path in csv_paths:
        means, _, _ = counter_means(path)
        for (k, c), (v, n) in means.items():
            if pat.search(k):
                names.add(k)
                vals[c] = v
        ds = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if pat.search(_short(r["Kernel_Name"])):
                ds[r["Counter_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        for c, v in ds.items():
            dur[c] = sum(v) / len(v)
    lines = [f"# Counters of {kernel} ({', '.join(sorted(names))}), workload {workload}", ""]
    for i, c in enumerate(cmds):
        lines += [f"Run {i + 1}:", "", "    " + c, ""]
    lines += [NOTE, "", "| counter | mean per dispatch |", "|---|---:|"]
    for c in sorted(vals):
        lines.append(f"| `{c}` | {vals[c]:.4g} |")
    derived = []
    if "GRBM_GUI_ACTIVE" in vals and dur.get("GRBM_GUI_ACTIVE"):
        d = dur["GRBM_GUI_ACTIVE"]
        derived.append(f"shader clock: {vals['GRBM_GUI_ACTIVE'] / 8 / d / 1e9:.2f} GHz "
                       f"(GRBM_GUI_ACTIVE / 8 XCDs / {d * 1e6:.1f} us dispatch, profiled)")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "SQ_BUSY_CU_CYCLES" in vals:
        derived.append(f"MFMA busy per busy CU cycle: {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / vals['SQ_BUSY_CU_CYCLES']:.3f}"
                       " (SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES)")
    if "SQ_INSTS_VALU" in vals and "SQ_INSTS_MFMA" in vals:
        derived.append(f"VALU instructions per MFMA: {vals['SQ_INSTS_VALU'] / max(vals['SQ_INSTS_MFMA'], 1):.2f}")
    if "SQ_INSTS_LDS" in vals and "SQ_INSTS_MFMA" in vals:
        derived.append(f"LDS instructions per MFMA: {vals['SQ_INSTS_LDS'] / max(vals['SQ_INSTS_MFMA'], 1):.2f}")
    if derived:
        lines += ["", "Derived:", ""] + [f"- {d}" for d in derived]
    lines += ["", f"sources_sha256: {sources_digest(kernel)}"]
    return "\n".join(lines) + "\n"


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")


def load_traffic(kernel: str, workload: str):
    """Calibrated HBM bytes per launch from the committed summary, or None when
    there is none or the kernel's sources have changed since it was taken."""
    p = traffic_path(kernel, workload)
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        m = re.match(r"^(\w+): (.*)$", line.strip())
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("sources_sha256") != sources_digest(kernel):
        return None
    return {"bytes": float(kv["traffic_bytes_per_launch"]),
            "fetch_bytes": float(kv["fetch_bytes_per_launch"]),
            "write_bytes": float(kv["write_bytes_per_launch"])}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", default="rocprofv3 kernel statistics")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--kernel", required=True, choices=sorted(KERNELS))
    b.add_argument("--workload", required=True)
    b.add_argument("--copy-mib", type=float, required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True, choices=sorted(KERNELS))
    c.add_argument("--workload", required=True)
    c.add_argument("--cmd", action="append", required=True)
    args = ap.parse_args(argv)
    if args.cmd_name == "stats":
        sys.stdout.write(format_stats(kernel_stats(args.csv), args.cmd, args.title))
    elif args.cmd_name == "counters":
        sys.stdout.write(counters_summary(args.csv, args.kernel, args.workload, args.cmd))
    else:
        sys.stdout.write(traffic_summary(args.fetch_csv, args.write_csv, args.kernel, args.workload,
                                         args.copy_mib, args.cmd_fetch, args.cmd_write))


if __name__ == "__main__":
    main()
