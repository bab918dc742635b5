"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/,
and read the HBM traffic figures back for the bench.

Three kinds of summary:

* ``trace``: the per-kernel table of ``rocprofv3 --kernel-trace --stats``
  (``*_kernel_stats.csv``): calls, average / min / max duration.
* ``mfma``: MFMA busy fraction and executed bf16 flops per launch of the
  verify kernels (one counter run).
* ``counters``: the mean per dispatch of any counters of one run, per
  library kernel (instruction mix, LDS use, waves).
* ``traffic``: HBM bytes per launch of each library kernel from two counter
  runs (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, KiB per dispatch), each
  scaled by what the same counter reads for a plain 1 GiB device copy
  (``bench.py --calibrate-copy``).  The factor is copy bytes / counter bytes.
  Each kernel's record carries a hash of its sources, so a figure taken on an
  older version of a kernel is not reported for the current one.

usage:
  python -m gated_deltanet_tree_03_amd.profiling trace STATS_CSV OUT --command CMD
  python -m gated_deltanet_tree_03_amd.profiling counters WORKLOAD OUT --counters DIR --command CMD
  python -m gated_deltanet_tree_03_amd.profiling traffic WORKLOAD OUT \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --command CMD [...] \\
      [--only KERNEL ...]
  python -m gated_deltanet_tree_03_amd.profiling mfma WORKLOAD OUT --counters DIR --command CMD
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from typing import Dict, List, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(PKG_DIR, "csrc")

# library kernel -> (substring of the device kernel name, its source files)
KERNELS = {
    "treewy_verify": ("verify_kernel", ["verify_kernel.h", "verify.hip"]),
    "treewy_commit_verify": ("verify_kernel", ["verify_kernel.h", "verify_fused.hip"]),
    "treewy_commit_verify_pool": ("verify_kernel", ["verify_kernel.h", "verify_pool.hip"]),
    "treewy_commit_verify_pool_trees": ("verify_kernel", ["verify_kernel.h", "verify_pool_trees.hip"]),
    "treewy_commit_verify_bf16state": ("verify_kernel", ["verify_kernel.h", "verify_s16.hip"]),
    "treewy_commit_verify_bf16state_pool": ("verify_kernel", ["verify_kernel.h", "verify_s16_pool.hip"]),
    "treewy_commit_verify_bf16state_pool_trees": ("verify_kernel", ["verify_kernel.h",
                                                                    "verify_s16_pool_trees.hip"]),
    "treewy_commit": ("commit_kernel", ["commit.hip"]),
    "treewy_store_all": ("store_all_kernel", ["store_all.hip"]),
    "treewy_store_all_select": ("select_kernel", ["store_all.hip"]),
    "treewy_prefill": ("prefill_kernel", ["verify_kernel.h", "prefill.hip"]),
}


def library_kernel(device_name: str) -> Optional[str]:
    """Library entry point whose kernel this device kernel name is, or None.
    The verify kernel's fourth template argument tells whether it also commits
    the previous step (treewy_commit_verify), the fifth whether the state sits
    in a slot-indexed pool (treewy_commit_verify_pool), the sixth whether it is
    stored as bf16 (treewy_commit_verify_bf16state), the seventh whether each
    sequence has its own tree (treewy_commit_verify_pool_trees); a bf16 state
    in a pool, with or without a tree per sequence, is
    treewy_commit_verify_bf16state_pool(_trees)."""
    if "verify_kernel<" in device_name:
        targs = [t.strip() for t in
                 device_name.split("verify_kernel<", 1)[1].split(">", 1)[0].split(",")]
        pool = len(targs) > 4 and targs[4] == "true"
        s16 = len(targs) > 5 and targs[5] == "true"
        ragged = len(targs) > 6 and targs[6] == "true"
        if s16:
            return ("treewy_commit_verify_bf16state_pool_trees" if ragged else
                    "treewy_commit_verify_bf16state_pool" if pool else "treewy_commit_verify_bf16state")
        if ragged:
            return "treewy_commit_verify_pool_trees"
        if pool:
            return "treewy_commit_verify_pool"
        return "treewy_commit_verify" if targs[3] == "true" else "treewy_verify"
    for k, (sub, _) in KERNELS.items():
        if sub in device_name and sub != "verify_kernel":
            return k
    return None
COMMON_SOURCES = ["device_common.h", "treewy_internal.h"]
COPY_BYTES = 2 ** 30  # bench.py --calibrate-copy: 1 GiB read + 1 GiB written per copy


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def source_sha(kernel: str) -> str:
    """Hash of the kernel's sources with comments and whitespace removed, so
    that an edit to comments alone keeps its counter records."""
    h = hashlib.sha256()
    for f in KERNELS[kernel][1] + COMMON_SOURCES:
        with open(os.path.join(CSRC, f)) as fh:
            code = _COMMENT.sub(" ", fh.read())
        h.update("".join(code.split()).encode())
    return h.hexdigest()[:16]


def _rows(path_or_dir: str, suffix: str) -> List[dict]:
    if os.path.isdir(path_or_dir):
        files = glob.glob(os.path.join(path_or_dir, "**", f"*{suffix}"), recursive=True)
    else:
        files = [path_or_dir]
    rows: List[dict] = []
    for f in sorted(files):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise FileNotFoundError(f"no *{suffix} rows under {path_or_dir}")
    return rows


def counter_means(path_or_dir: str, counter: str) -> Dict[str, float]:
    """Mean counter value per dispatch (KiB for FETCH_SIZE / WRITE_SIZE), keyed
    by library kernel name, plus '__copy__' for the device copy kernel."""
    sums: Dict[str, List[float]] = {}
    for r in _rows(path_or_dir, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        key = library_kernel(name)
        if key is None and "copyBuffer" in name:
            key = "__copy__"
        if key is None:
            continue
        sums.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in sums.items()}


def traffic(workload: str, fetch: str, write: str, copy_fetch: str, copy_write: str,
            out: str, commands: List[str], only: Optional[List[str]] = None) -> List[dict]:
    """`only`: record just these library kernels (a run whose other kernels
    are not the workload's own, e.g. the prefill run)."""
    f = counter_means(fetch, "FETCH_SIZE")
    w = counter_means(write, "WRITE_SIZE")
    cf = counter_means(copy_fetch, "FETCH_SIZE")["__copy__"]
    cw = counter_means(copy_write, "WRITE_SIZE")["__copy__"]
    fetch_scale = COPY_BYTES / (cf * 1024.0)
    write_scale = COPY_BYTES / (cw * 1024.0)
    recs = []
    for k in KERNELS:
        if k not in f or k not in w or (only and k not in only):
            continue
        rd = f[k] * 1024.0 * fetch_scale
        wr = w[k] * 1024.0 * write_scale
        recs.append({"kernel": k, "workload": workload, "fetch_kib_raw": round(f[k], 1),
                     "write_kib_raw": round(w[k], 1), "fetch_scale": round(fetch_scale, 4),
                     "write_scale": round(write_scale, 4), "hbm_read_bytes": int(rd),
                     "hbm_write_bytes": int(wr), "hbm_bytes_per_launch": int(rd + wr),
                     "source_sha": source_sha(k)})
    lines = [f"# HBM traffic per launch, workload {workload}", "",
             "Counters: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the",
             "dispatches of the run), each scaled by copy bytes / counter bytes of a plain",
             f"1 GiB device copy (copy FETCH_SIZE {cf:.1f} KiB -> factor {fetch_scale:.4f};",
             f"copy WRITE_SIZE {cw:.1f} KiB -> factor {write_scale:.4f}).", "",
             "Commands (run from /tmp with TMPDIR=/tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | write bytes | total bytes |",
              "|---|---|---|---|---|---|"]
    for r in recs:
        lines.append(f"| {r['kernel']} | {r['fetch_kib_raw']} | {r['write_kib_raw']} | "
                     f"{r['hbm_read_bytes']} | {r['hbm_write_bytes']} | {r['hbm_bytes_per_launch']} |")
    lines += ["", "Machine-readable records (one per kernel; source_sha identifies the kernel",
              "sources the counters were taken on):", ""]
    lines += ["    " + json.dumps(r) for r in recs]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return recs


def read_traffic(kernel: str, workload: str) -> Optional[int]:
    """HBM bytes per launch of `kernel` on `workload` from the committed
    summary, or None if absent or taken on different kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if not line.startswith("{"):
            continue
        rec = json.loads(line)
        if rec.get("kernel") == kernel and rec.get("workload") == workload:
            if rec.get("source_sha") != source_sha(kernel):
                return None
            return int(rec["hbm_bytes_per_launch"])
    return None


MFMA_PEAK_BF16 = 2.5e15  # dense bf16 MFMA flop/s of MI355X
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9


def _dispatches(path_or_dir: str) -> Dict[str, dict]:
    """Per dispatch of a library kernel: its counters and duration (ns, from
    the dispatch's start and end timestamps)."""
    out: Dict[str, dict] = {}
    for r in _rows(path_or_dir, "counter_collection.csv"):
        key = library_kernel(r["Kernel_Name"])
        if key is None:
            continue
        d = out.setdefault(r["Dispatch_Id"], {"kernel": key, "ns": 0.0})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def mfma(workload: str, counters: str, out: str, commands: List[str]) -> List[dict]:
    """MFMA use of the verify kernels from one counter run with
    SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_BF16.  Busy % =
    MFMA-busy SIMD cycles / (dispatch duration x clock x SIMDs).  Executed
    flops = MOPS x 512.  The algorithmic contraction is S0 [K;Q] (4 d^2 N
    flops per head); execution adds the bf16 hi/lo split of S0 (x2), padding
    of 2N rows to 16-row tiles and the [K;Q] K^T gram.  Durations under
    counter collection run longer than unprofiled ones, so the rates here are
    lower bounds."""
    from . import synth
    cfg = synth.CONFIGS[workload]
    N = len(cfg.parent)
    algo = 4.0 * 128 * 128 * N * cfg.B * cfg.H
    per: Dict[str, List[dict]] = {}
    for d in _dispatches(counters).values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in d and d["ns"] > 0:
            per.setdefault(d["kernel"], []).append(d)
    recs = []
    for k in KERNELS:
        ds = per.get(k, [])
        if not ds:
            continue
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / len(ds)
        flops = 512.0 * sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds) / len(ds)
        secs = sum(d["ns"] for d in ds) / len(ds) * 1e-9
        if flops <= 0:
            continue
        recs.append({"kernel": k, "workload": workload, "dispatches": len(ds),
                     "mfma_busy_pct": round(100.0 * busy / (secs * CLOCK_HZ * SIMDS), 2),
                     "executed_flops": int(flops), "algorithmic_flops": int(algo),
                     "profiled_us": round(secs * 1e6, 2),
                     "executed_tflops": round(flops / secs / 1e12, 1),
                     "pct_of_bf16_peak": round(100.0 * flops / secs / MFMA_PEAK_BF16, 2),
                     "source_sha": source_sha(k)})
    lines = [f"# MFMA use per launch, workload {workload}", "",
             "Counters: rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_BF16, per",
             "dispatch, with the dispatch's start/end timestamps (means over the run).",
             f"busy % = MFMA-busy SIMD cycles / (duration x {CLOCK_HZ / 1e9:.1f} GHz x {SIMDS} SIMDs);",
             "executed flops = MOPS x 512; peak = 2.5 PFLOP/s dense bf16.  Profiled durations are",
             "longer than unprofiled ones, so rates are lower bounds.",
             f"Algorithmic contraction S0.[K;Q] = 4 d^2 N flops per head = {algo:.4g} per launch.", "",
             "Command (run from /tmp with TMPDIR=/tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "| kernel | MFMA busy % | executed flops | algorithmic flops | profiled us | TFLOP/s | % of bf16 peak |",
              "|---|---|---|---|---|---|---|"]
    for r in recs:
        lines.append(f"| {r['kernel']} | {r['mfma_busy_pct']} | {r['executed_flops']:.4g} | "
                     f"{r['algorithmic_flops']:.4g} | {r['profiled_us']} | {r['executed_tflops']} | "
                     f"{r['pct_of_bf16_peak']} |")
    lines += ["", "Machine-readable records:", ""]
    lines += ["    " + json.dumps(r) for r in recs]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return recs


def counters(workload: str, path: str, out: str, commands: List[str], title: str) -> List[dict]:
    """Mean value per dispatch of every counter of one counter run, per
    library kernel, with the mean dispatch duration under the counters."""
    per: Dict[str, List[dict]] = {}
    for d in _dispatches(path).values():
        per.setdefault(d["kernel"], []).append(d)
    recs = []
    names: List[str] = []
    for k in KERNELS:
        ds = per.get(k, [])
        if not ds:
            continue
        cs = sorted({c for d in ds for c in d if c not in ("kernel", "ns")})
        names = sorted(set(names) | set(cs))
        rec = {"kernel": k, "workload": workload, "dispatches": len(ds),
               "profiled_us": round(sum(d["ns"] for d in ds) / len(ds) / 1e3, 2)}
        for c in cs:
            rec[c] = round(sum(d.get(c, 0.0) for d in ds) / len(ds), 1)
        rec["source_sha"] = source_sha(k)
        recs.append(rec)
    lines = [f"# {title}", "", "Counters: rocprofv3 --pmc, mean value per dispatch over the run "
             "(profiled durations run longer than unprofiled ones).", "",
             "Command (run from /tmp with TMPDIR=/tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "| kernel | dispatches | profiled us | " + " | ".join(names) + " |",
              "|---|---|---|" + "---|" * len(names)]
    for r in recs:
        lines.append(f"| {r['kernel']} | {r['dispatches']} | {r['profiled_us']} | " +
                     " | ".join(f"{r.get(c, 0):.4g}" for c in names) + " |")
    lines += ["", "Machine-readable records:", ""]
    lines += ["    " + json.dumps(r) for r in recs]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return recs


def trace(stats_csv: str, out: str, commands: List[str], title: str) -> None:
    rows = _rows(stats_csv, "kernel_stats.csv")
    lines = [f"# {title}", "", "Command (run from /tmp with TMPDIR=/tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "| kernel | calls | average us | min us | max us | % of GPU time |",
              "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = name.replace("void ", "").replace("treewy::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out")
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--title", default="rocprofv3 kernel trace")
    r = sub.add_parser("traffic")
    r.add_argument("workload")
    r.add_argument("out")
    for opt in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        r.add_argument(opt, required=True)
    r.add_argument("--command", action="append", default=[])
    r.add_argument("--only", action="append", default=None, help="record only this kernel")
    m = sub.add_parser("mfma")
    m.add_argument("workload")
    m.add_argument("out")
    m.add_argument("--counters", required=True)
    m.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("workload")
    c.add_argument("out")
    c.add_argument("--counters", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--title", default="rocprofv3 counters")
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        for rec in counters(a.workload, a.counters, a.out, a.command, a.title):
            print(json.dumps(rec))
    elif a.cmd == "trace":
        trace(a.stats_csv, a.out, a.command, a.title)
    elif a.cmd == "mfma":
        for rec in mfma(a.workload, a.counters, a.out, a.command):
            print(json.dumps(rec))
    else:
        for rec in traffic(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write, a.out, a.command,
                           a.only):
            print(json.dumps(rec))


if __name__ == "__main__":
    sys.exit(main())
