"""Offline tile tuning of the fused 16-bit attention kernel.

The WebGPU page ("WebGPU 算子优化…", section "浏览器端落地的关键参数与监控")
picks the sequence and head-dimension tile sizes per device with a probe at
the first run, falling back to smaller tiles when the shared-memory
allocation fails. On gfx950 every candidate is known at compile time, so the
choice moves offline: libattn compiles a few tile variants per head size
(``attn_fwd_tile_info`` lists them), this script times each of them on the
target GPU over a grid of shapes, and writes the fastest per grid cell to
``csrc/tile_table.inc``, which ``attn_fwd`` consults after a rebuild.

Grid: query rows B*H*Sq = 2^12 .. 2^20 and key lengths Sk = 2^8 .. 2^14
(a call is placed in the cell of the nearest powers of two), per head size
(64, 128) and masking (none, causal). Each cell is timed on bf16 inputs with
B = 1, Sq = min(Sk, rows) and H = rows / Sq; fp16 runs the same tiles and
takes the same choice.

Usage, on the GPU the table is for::

    python -m scaled_dot_product_flashattention_amd.autotune [--json timings.json]
    python -m scaled_dot_product_flashattention_amd.build
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics

ROWS_LOG2_MIN, ROWS_BUCKETS = 12, 9
KEYS_LOG2_MIN, KEYS_BUCKETS = 8, 7
HEADS = (64, 128)
# another variant replaces variant 0 only when it is this much faster, so
# that timing noise does not move cells where the variants tie
MARGIN = 0.03
TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "tile_table.inc")


def cells():
    """(d index, causal, rows bucket, keys bucket, B, H, Sq, Sk) of the grid."""
    for di, d in enumerate(HEADS):
        for causal in (0, 1):
            for ri in range(ROWS_BUCKETS):
                rows = 1 << (ROWS_LOG2_MIN + ri)
                for ki in range(KEYS_BUCKETS):
                    sk = 1 << (KEYS_LOG2_MIN + ki)
                    sq = min(sk, rows)
                    yield di, d, causal, ri, ki, 1, rows // sq, sq, sk


def rule_table():
    """The choice before tuning: two key halves (variant 2) for head size 64
    from 2048 keys on, variant 0 otherwise."""
    t = [[[[0] * KEYS_BUCKETS for _ in range(ROWS_BUCKETS)] for _ in range(2)] for _ in range(2)]
    for ri in range(ROWS_BUCKETS):
        for ki in range(KEYS_BUCKETS):
            if KEYS_LOG2_MIN + ki >= 11:
                t[0][0][ri][ki] = t[0][1][ri][ki] = 2
    return t


def write_table(table, source: str, gain=None, path: str = TABLE_PATH) -> None:
    """Write the table as C++ (included by the 16-bit kernel's source).
    ``gain[di][c][ri][ki]`` is the chosen variant's speed-up over variant 0."""
    lines = [
        "// Tile variant of the fused 16-bit attention kernel per grid cell.",
        f"// Written by scaled_dot_product_flashattention_amd/autotune.py ({source}).",
        "// Regenerate on the target GPU with that script and rebuild; do not edit.",
        f"// Cells: query rows B*H*Sq = 2^{ROWS_LOG2_MIN} .. 2^{ROWS_LOG2_MIN + ROWS_BUCKETS - 1}, key length "
        f"2^{KEYS_LOG2_MIN} .. 2^{KEYS_LOG2_MIN + KEYS_BUCKETS - 1}",
        "// (nearest power of two, clamped). Comments give the chosen variant's",
        "// speed-up over variant 0 where measured.",
        f"constexpr int kTuneRowsLog2Min = {ROWS_LOG2_MIN};",
        f"constexpr int kTuneRowsBuckets = {ROWS_BUCKETS};",
        f"constexpr int kTuneKeysLog2Min = {KEYS_LOG2_MIN};",
        f"constexpr int kTuneKeysBuckets = {KEYS_BUCKETS};",
        "// kTileTable[head size 64, 128][not causal, causal][rows][keys]",
        "const signed char kTileTable[2][2][kTuneRowsBuckets][kTuneKeysBuckets] = {",
    ]
    for di, d in enumerate(HEADS):
        lines.append(f"    {{  // head size {d}")
        for c in (0, 1):
            lines.append(f"        {{  // {'causal' if c else 'no mask'}")
            for ri in range(ROWS_BUCKETS):
                row = ", ".join(str(v) for v in table[di][c][ri])
                note = ""
                if gain is not None:
                    note = "  x" + " ".join(f"{g:.2f}" for g in gain[di][c][ri])
                lines.append(f"            {{{row}}},  // rows 2^{ROWS_LOG2_MIN + ri}{note}")
            lines.append("        },")
        lines.append("    },")
    lines.append("};")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _time_variants(sdpa, torch, q, k, v, o, lse, causal, n_var):
    """Median time (ms) per launch of each variant, rounds interleaved."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def run(t, n):
        for _ in range(n):
            sdpa.attn_fwd_tiled(q, k, v, tile=t, causal=bool(causal), out=o, lse=lse)

    for t in range(n_var):
        run(t, 3)
    torch.cuda.synchronize()
    ev[0].record()
    run(0, 3)
    ev[1].record()
    torch.cuda.synchronize()
    est = max(ev[0].elapsed_time(ev[1]) / 3, 1e-3)
    n = max(10, min(2000, math.ceil(3.0 / est)))  # about 3 ms per batch
    samples = [[] for _ in range(n_var)]
    for _ in range(7):
        for t in range(n_var):
            ev[0].record()
            run(t, n)
            ev[1].record()
            torch.cuda.synchronize()
            samples[t].append(ev[0].elapsed_time(ev[1]) / n)
    return [statistics.median(s) for s in samples]


def measure(verbose=True) -> dict:
    """One timing pass over the grid on cuda:0: every variant in every cell."""
    import torch

    import scaled_dot_product_flashattention_amd as sdpa

    if not torch.cuda.is_available():
        raise SystemExit("tile tuning needs the GPU the table is for")
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    arch = getattr(props, "gcnArchName", "").split(":")[0]
    device = f"{arch or props.name}, {props.multi_processor_count} CUs"
    record = {"device": device, "cells": []}
    gen = torch.Generator(device=dev)
    for di, d, causal, ri, ki, B, H, Sq, Sk in cells():
        gen.manual_seed(1000 * di + 100 * causal + 10 * ri + ki)
        q = torch.randn((B, H, Sq, d), generator=gen, device=dev, dtype=torch.bfloat16)
        k = torch.randn((B, H, Sk, d), generator=gen, device=dev, dtype=torch.bfloat16)
        v = torch.randn((B, H, Sk, d), generator=gen, device=dev, dtype=torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Sq), device=dev, dtype=torch.float32)
        n_var = sdpa.attn_fwd_tile_count(d, torch.bfloat16)
        ms = _time_variants(sdpa, torch, q, k, v, o, lse, causal, n_var)
        record["cells"].append({"d": d, "causal": causal, "rows_bucket": ri, "keys_bucket": ki,
                                "B": B, "H": H, "Sq": Sq, "Sk": Sk, "ms": ms})
        if verbose:
            print(f"d{d} causal={causal} H{H} Sq{Sq} Sk{Sk}: " +
                  " ".join(f"{t}:{m * 1e3:.1f}us" for t, m in enumerate(ms)), flush=True)
        del q, k, v, o, lse
    return record


def choose(records):
    """The table from one or more passes: per cell, the variant with the
    lowest mean time over the passes; another variant than 0 only when it
    beats variant 0 by MARGIN."""
    table = [[[[0] * KEYS_BUCKETS for _ in range(ROWS_BUCKETS)] for _ in range(2)] for _ in range(2)]
    gain = [[[[1.0] * KEYS_BUCKETS for _ in range(ROWS_BUCKETS)] for _ in range(2)] for _ in range(2)]
    for cs in zip(*(r["cells"] for r in records)):
        c0 = cs[0]
        key = (c0["d"], c0["causal"], c0["Sq"], c0["Sk"], c0["H"])
        if any((c["d"], c["causal"], c["Sq"], c["Sk"], c["H"]) != key for c in cs):
            raise ValueError("passes over different grids")
        n_var = len(c0["ms"])
        mean = [statistics.fmean(c["ms"][t] for c in cs) for t in range(n_var)]
        best = min(range(n_var), key=lambda t: mean[t])
        if best != 0 and mean[best] > (1.0 - MARGIN) * mean[0]:
            best = 0
        di, ri, ki = HEADS.index(c0["d"]), c0["rows_bucket"], c0["keys_bucket"]
        table[di][c0["causal"]][ri][ki] = best
        gain[di][c0["causal"]][ri][ki] = mean[0] / mean[best]
    return table, gain


def main() -> int:
    ap = argparse.ArgumentParser(description="time the fused kernel's tile variants and "
                                             "write csrc/tile_table.inc")
    ap.add_argument("--passes", type=int, default=2, help="timing passes over the grid")
    ap.add_argument("--json", default=None, help="also write every pass's timings to this file")
    ap.add_argument("--from-json", nargs="+", default=None,
                    help="derive the table from timing files written by --json (no GPU)")
    ap.add_argument("--out", default=TABLE_PATH, help="where to write the table")
    ap.add_argument("--rule", action="store_true",
                    help="write the untuned rule instead of timing (no GPU needed)")
    args = ap.parse_args()
    if args.rule:
        write_table(rule_table(), "untuned rule", path=args.out)
        return 0
    if args.from_json:
        records = []
        for f in args.from_json:
            with open(f) as fh:
                rec = json.load(fh)
            records.extend(rec["passes"] if "passes" in rec else [rec])
    else:
        records = [measure() for _ in range(args.passes)]
        if args.json:
            with open(args.json, "w") as fh:
                json.dump({"margin": MARGIN, "passes": records}, fh, indent=1)
    devices = sorted({r["device"] for r in records})
    table, gain = choose(records)
    write_table(table, f"mean of {len(records)} timing passes on {' / '.join(devices)}", gain,
                args.out)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
