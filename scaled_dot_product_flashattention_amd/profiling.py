"""Summaries of rocprofv3 results (rocpd SQLite databases) as short text.

Used to keep the measured figures behind bench.py's roofline under profiles/:

* kernel-trace summary: per kernel, dispatch count and mean / min / max
  duration, from a ``rocprofv3 --kernel-trace --stats`` run;
* shader clock under one kernel: GRBM_GUI_ACTIVE cycles per dispatch over
  the dispatch's duration, from a ``rocprofv3 --pmc GRBM_GUI_ACTIVE`` run;
* HBM traffic: per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of one kernel from
  two ``rocprofv3 --pmc`` runs, each scaled by what the same counter reads for a
  plain device copy of known size in the same run (bench.py --copy-calibration
  runs three 256 MiB copies).

    python -m scaled_dot_product_flashattention_amd.profiling trace DB OUT.md --command "..." \
        [--timed STEPS --bench-log LOG]
    python -m scaled_dot_product_flashattention_amd.profiling traffic FETCH_DB WRITE_DB \
        --kernel fwd_prefill_kernel --workload medium_bf16 --path fused --command "..."
    python -m scaled_dot_product_flashattention_amd.profiling clock GRBM_DB \
        --kernel fwd_prefill16_kernel --workload medium_bf16 --path fused --command "..."
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20
COPY_KERNEL = "copyBuffer"


def kernel_trace(db_path: str):
    db = sqlite3.connect(db_path)
    rows = db.execute(
        "select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    return [dict(name=r[0], calls=r[1], avg_ns=r[2], min_ns=r[3], max_ns=r[4], total_ns=r[5])
            for r in rows]


def counter_per_kernel(db_path: str, counter: str):
    db = sqlite3.connect(db_path)
    rows = db.execute(
        "select kernel_name, count(*), avg(value), avg(duration) from counters_collection "
        "where counter_name = ? group by kernel_name", (counter,)).fetchall()
    return {r[0]: dict(dispatches=r[1], kib=r[2], avg_ns=r[3]) for r in rows}


def _pick(per_kernel: dict, needle: str):
    hits = [(k, v) for k, v in per_kernel.items() if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {[k for k, _ in hits]}")
    return hits[0]


def kernel_kind(kernel_name: str) -> str:
    """Which source family a kernel comes from: fused, splitk, naive, qkv or softmax."""
    if "splitk" in kernel_name:
        return "splitk"
    if "naive" in kernel_name:
        return "naive"
    if "qkv_proj" in kernel_name:
        return "qkv"
    if "softmax_" in kernel_name:
        return "softmax"
    return "fused"


def source_digest(kind: str) -> str:
    """sha256 over the sources of one kernel family (see kernel_kind)."""
    csrc = os.path.join(ROOT, "scaled_dot_product_flashattention_amd", "csrc")
    files = {"fused": ["fwd_prefill.hip", "fwd_prefill16.hip", "tile_table.inc", "device_common.h"],
             "splitk": ["fwd_splitk.hip", "device_common.h"],
             "naive": ["naive.hip", "device_common.h"],
             "qkv": ["qkv_proj.hip", "device_common.h"],
             "softmax": ["softmax_rows.hip", "device_common.h"]}[kind]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f)) as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()


def code_only(src: str) -> str:
    """C/C++ source without comments and blank lines, so that an edit of a
    comment does not count as a change of the kernel."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def timed_means(db_path: str, last: int):
    """Per kernel, the mean duration (ns) of its last ``last`` dispatches in
    start order: the dispatches of bench.py's timed region."""
    db = sqlite3.connect(db_path)
    by: dict[str, list[int]] = {}
    for name, start, end in db.execute("select name, start, end from kernels order by start"):
        by.setdefault(name, []).append(end - start)
    return {n: sum(d[-last:]) / last for n, d in by.items() if len(d) >= last}


def write_trace(db_path: str, out_md: str, command: str, timed: int = 0,
                bench_line: str | None = None) -> None:
    ks = kernel_trace(db_path)
    tm = timed_means(db_path, timed) if timed else {}
    lines = ["# Kernel trace summary", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | mean us | min us | max us | total us |"
             + (f" mean of last {timed} us |" if timed else ""),
             "|---|---|---|---|---|---|" + ("---|" if timed else "")]
    for k in ks:
        row = (f"| `{k['name'][:110]}` | {k['calls']} | {k['avg_ns'] / 1e3:.2f} | "
               f"{k['min_ns'] / 1e3:.2f} | {k['max_ns'] / 1e3:.2f} | {k['total_ns'] / 1e3:.1f} |")
        if timed:
            row += f" {tm[k['name']] / 1e3:.2f} |" if k["name"] in tm else " - |"
        lines.append(row)
    if timed:
        lines += ["", f"The last {timed} dispatches of a kernel are the ones bench.py times "
                  "(its warmup dispatches come first)."]
    if bench_line:
        rec = json.loads(bench_line)
        lines += ["", f"bench.py in the same run: {rec['value']} {rec['unit']}, "
                  f"{rec['ms_per_step'] * 1e3:.2f} us per step (HIP events over the timed region)."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(fetch_db: str, write_db: str, kernel: str, workload: str, path: str,
                  command: str) -> dict:
    fetch = counter_per_kernel(fetch_db, "FETCH_SIZE")
    write = counter_per_kernel(write_db, "WRITE_SIZE")
    kname, kf = _pick(fetch, kernel)
    _, kw = _pick(write, kernel)
    _, cf = _pick(fetch, COPY_KERNEL)
    _, cw = _pick(write, COPY_KERNEL)
    f_scale = COPY_BYTES / (cf["kib"] * 1024.0)
    w_scale = COPY_BYTES / (cw["kib"] * 1024.0)
    fetch_b = kf["kib"] * 1024.0 * f_scale
    write_b = kw["kib"] * 1024.0 * w_scale
    rec = {
        "workload": workload,
        "path": path,
        "kernel": kname,
        "kernel_source_sha256": source_digest(kernel_kind(kname)),
        "fetch_kib_per_dispatch": kf["kib"],
        "write_kib_per_dispatch": kw["kib"],
        "copy_fetch_kib": cf["kib"],
        "copy_write_kib": cw["kib"],
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_fetch_bytes_per_launch": fetch_b,
        "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "command": command,
    }
    base = os.path.join(PROFILES, f"{workload}_{path}_traffic")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic: {workload}, {path} path", "", "Commands (one counter per run):", "",
             "```", command, "```", "",
             f"Kernel: `{kname[:120]}`", "",
             "| counter | KiB / dispatch | copy of 256 MiB reads | scale | bytes / launch |",
             "|---|---|---|---|---|",
             f"| FETCH_SIZE | {kf['kib']:.1f} | {cf['kib']:.1f} KiB | {f_scale:.4f} | {fetch_b:.4e} |",
             f"| WRITE_SIZE | {kw['kib']:.1f} | {cw['kib']:.1f} KiB | {w_scale:.4f} | {write_b:.4e} |",
             "", f"Total HBM bytes per launch: {fetch_b + write_b:.4e}",
             f"Kernel source sha256 ({kernel_kind(kname)} kernel files): {rec['kernel_source_sha256']}"]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    return rec


def write_clock(db_path: str, kernel: str, workload: str, path: str, command: str,
                xccs: int = 8) -> dict:
    """Shader clock under the kernel from a ``rocprofv3 --pmc GRBM_GUI_ACTIVE``
    run: the counter (GPU-busy cycles, summed over the XCCs) per dispatch,
    divided by the XCC count and by the dispatch's duration."""
    per = counter_per_kernel(db_path, "GRBM_GUI_ACTIVE")
    kname, k = _pick(per, kernel)
    cycles = k["kib"] / xccs  # counter_per_kernel's "kib" is the counter's mean value
    mhz = cycles / (k["avg_ns"] * 1e-9) / 1e6
    rec = {"workload": workload, "path": path, "kernel": kname,
           "kernel_source_sha256": source_digest(kernel_kind(kname)),
           "grbm_gui_active_per_dispatch": k["kib"], "xccs": xccs,
           "cycles_per_dispatch": cycles, "avg_ns_under_counters": k["avg_ns"],
           "dispatches": k["dispatches"], "gfx_mhz": mhz, "command": command}
    base = os.path.join(PROFILES, f"{workload}_{path}_clock")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# Shader clock under the kernel: {workload}, {path} path", "", "Command:", "",
             "```", command, "```", "", f"Kernel: `{kname[:120]}`", "",
             "| GRBM_GUI_ACTIVE per dispatch (sum over XCCs) | XCCs | cycles | mean duration | clock |",
             "|---|---|---|---|---|",
             f"| {k['kib']:.0f} | {xccs} | {cycles:.0f} | {k['avg_ns'] / 1e3:.2f} us | {mhz:.0f} MHz |",
             "", f"Kernel source sha256 ({kernel_kind(kname)} kernel files): {rec['kernel_source_sha256']}"]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    return rec


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--timed", type=int, default=0,
                   help="also average each kernel's last N dispatches (bench.py --steps N)")
    t.add_argument("--bench-log", default=None,
                   help="file holding bench.py's JSON line from the same run")
    r = sub.add_parser("traffic")
    r.add_argument("fetch_db")
    r.add_argument("write_db")
    r.add_argument("--kernel", required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--path", required=True)
    r.add_argument("--command", required=True)
    c = sub.add_parser("clock")
    c.add_argument("db")
    c.add_argument("--kernel", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--path", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "trace":
        line = None
        if a.bench_log:
            with open(a.bench_log) as f:
                line = [x for x in f.read().splitlines() if x.startswith("{")][-1]
        write_trace(a.db, a.out, a.command, a.timed, line)
    elif a.cmd == "clock":
        print(json.dumps(write_clock(a.db, a.kernel, a.workload, a.path, a.command), indent=1))
    else:
        print(json.dumps(write_traffic(a.fetch_db, a.write_db, a.kernel, a.workload, a.path,
                                       a.command), indent=1))


if __name__ == "__main__":
    main()
