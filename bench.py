"""Benchmark of the fused attention forward on one MI355X.

Default (no flags): the medium prefill workload, B=1 H=16 Sq=Sk=4096 d=64,
bf16, [B,H,S,d], non-causal, LSE out. One step = one attn_fwd call (the fused
kernel: Q tile load, K/V streaming, QK^T, mask, online softmax, PV, epilogue).
Prints one JSON line with the throughput in TFLOP/s, the roofline of the
fused kernel and the fp64 oracle timed on the host cores.

FLOPs per step: 4*B*H*Sq*Sk*d (two products of 2*d FLOPs per score), halved
for causal masks. Inputs are resident in HBM before the timed region.

Other workloads (--config) and the unfused baseline (--path naive) are for
the design notes; only the default line is the headline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS_16 = 2516.6   # MI355X dense bf16/fp16 matrix peak: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_TFLOPS_F32 = 157.3   # MI355X fp32 peak
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def flops(w) -> float:
    """Nominal FLOPs of one forward: 4*B*H*Sq*Sk*d, halved for causal masks."""
    f = 4.0 * w.B * w.H * w.Sq * w.Sk * w.d
    return f / 2 if w.causal else f


def valid_pairs(w, kv_len) -> float:
    """(query, key) pairs the method computes: keys below each sequence's
    length and, with a causal mask, keys j <= i."""
    import numpy as np

    lens = np.full(w.B, w.Sk, dtype=np.int64) if kv_len is None else \
        np.clip(np.asarray(kv_len, dtype=np.int64), 0, w.Sk)
    i = np.arange(w.Sq, dtype=np.int64)
    tot = sum(int(np.minimum(i + 1, n).sum()) if w.causal else w.Sq * int(n) for n in lens)
    return float(tot) * w.H


def algorithmic_flops(w, kv_len) -> float:
    """FLOPs credited to a step: the nominal count, except for key padding,
    where only the valid pairs count (4*d FLOPs each)."""
    return 4.0 * w.d * valid_pairs(w, kv_len) if w.kv_len_range is not None else flops(w)


def kv_bytes(w) -> float:
    es = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    return 2.0 * w.B * w.H * w.Sk * w.d * es


def stored_traffic(workload: str, path: str, kind: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    profile of this workload, or None when there is none or the kernel's
    source (family ``kind``: fused, splitk, naive) changed since."""
    fn = os.path.join(PROFILES, f"{workload}_{path}_traffic.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    from scaled_dot_product_flashattention_amd.profiling import source_digest

    if rec.get("kernel_source_sha256") != source_digest(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def stored_clock(workload: str, path: str, kind: str):
    """Shader clock (MHz) under the dominant kernel from the committed
    GRBM_GUI_ACTIVE profile of this workload, or None when there is none or
    the kernel's source changed since."""
    fn = os.path.join(PROFILES, f"{workload}_{path}_clock.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    from scaled_dot_product_flashattention_amd.profiling import source_digest

    if rec.get("kernel_source_sha256") != source_digest(kind):
        return None
    return rec.get("gfx_mhz")


def cpu_share() -> int:
    """Host threads for the oracle: OMP_NUM_THREADS where the machine sets it
    (a shared GPU machine allots its CPUs per GPU and says so there), else every
    CPU this process may run on."""
    import oracle

    return oracle.host_threads()


def output_rows(o, rows, w):
    """Rows (b*H + h)*Sq + i of the output o (any layout) as a float64 array."""
    import numpy as np

    o_c = o.float().cpu()
    out = np.empty((len(rows), w.d))
    for n, r in enumerate(rows):
        i, h, b = r % w.Sq, (r // w.Sq) % w.H, r // (w.Sq * w.H)
        if w.layout == "bhsd":
            out[n] = o_c[b, h, i].numpy()
        elif w.layout == "bshd":
            out[n] = o_c[b, i, h].numpy()
        else:
            g = o_c.shape[3]
            out[n] = o_c[b, h // g, i, h % g].numpy()
    return out


def timed_region(step, steps: int, stream, torch):
    """Run ``steps`` calls of ``step`` on ``stream`` between HIP events, in
    five equal batches (the last takes the remainder) with an event at each
    boundary. Returns the mean ms per step over the whole region and the
    per-step means of the batches."""
    nb = min(5, steps)
    sizes = [steps // nb + (1 if i < steps % nb else 0) for i in range(nb)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    ev[0].record(stream)
    for i, n in enumerate(sizes):
        for _ in range(n):
            step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[nb]) / steps
    batches = [ev[i].elapsed_time(ev[i + 1]) / sizes[i] for i in range(nb)]
    return total, batches


def prewarm(step, seconds: float, torch) -> int:
    """Run ``step`` until ``seconds`` of wall time have passed (the GPU's
    clock ramps up under load over tens of milliseconds; a handful of warmup
    steps of a 0.1 ms kernel would otherwise time the ramp). Returns the
    number of steps run."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            step()
        n += 50
        torch.cuda.synchronize()
    return n


def timing_summary(ms: float, batches) -> dict:
    srt = sorted(batches)
    return {"ms_mean": round(ms, 5), "ms_median_of_batches": round(srt[len(srt) // 2], 5),
            "ms_min_of_batches": round(srt[0], 5), "batches": len(batches)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, t, o=None, lse=None, target_s: float = 12.0):
    """The fp64 oracle on a bounded sample of rows of the same workload,
    timed on the host cores, scaled to the metric's unit. With the GPU's
    output (o, lse) of the same inputs, also the largest differences on
    those rows."""
    import numpy as np

    import oracle

    cores = cpu_share()
    R = w.B * w.H * w.Sq
    rng = np.random.default_rng(5)
    n = min(R, 4 * cores)
    while True:
        rows = np.sort(rng.choice(R, size=n, replace=False))
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention_rows(t["q"], t["k"], t["v"], rows, scale=w.scale,
                                               causal=w.causal, layout=w.layout,
                                               kv_len=t["kv_len"], nthreads=cores)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n >= R:
            break
        n = min(R, max(n * 2, int(n * target_s / max(dt, 1e-3))))
    # the pairs of the sampled rows
    lens = np.full(w.B, w.Sk) if t["kv_len"] is None else np.clip(t["kv_len"].numpy(), 0, w.Sk)
    i, b = rows % w.Sq, rows // (w.Sq * w.H)
    f = float(np.sum(4.0 * w.d * (np.minimum(i + 1, lens[b]) if w.causal else lens[b])))
    rec = {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(), "host_cpus_visible": os.cpu_count(),
           "wall_s": round(dt, 2), "gflops": round(f / dt / 1e9, 2),
           "full_workload_s_estimate": round(dt * valid_pairs(w, t["kv_len"]) * 4.0 * w.d / f, 1),
           "sample": f"{len(rows)} of {R} query rows of the same workload, full key range each, "
                     f"{dt:.1f} s wall on {cores} threads (fp64, three-step softmax)"}
    if o is not None:
        got = output_rows(o, rows, w)
        got_l = lse.cpu().numpy().reshape(-1)[rows].astype(np.float64)
        both_inf = np.isneginf(got_l) & np.isneginf(lse_ref)
        with np.errstate(invalid="ignore"):
            dl = np.where(both_inf, 0.0, np.abs(got_l - lse_ref))
        rec["gpu_max_abs_err"] = {"o": float(np.abs(got - o_ref).max()), "lse": float(dl.max()),
                                  "rows": len(rows)}
    return rec


def bench_softmax(args, w, torch, sdpa) -> int:
    """Row softmax over score-like rows shaped like the workload's score
    matrix: B*H*Sq rows of Sk, in the workload's dtype."""
    from scaled_dot_product_flashattention_amd.inputs import generate_softmax_rows

    rows, n = w.B * w.H * w.Sq, w.Sk
    dev = torch.device("cuda:0")
    x = generate_softmax_rows(rows, n, w.dtype, seed=w.seed).to(dev)
    y = torch.empty_like(x)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    mode = args.path[len("softmax_"):]
    step = lambda: sdpa.attn_softmax_rows(x, scale=w.scale, mode=mode, out=y, lse=lse)  # noqa: E731
    prewarm(step, args.prewarm_s, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ms, batches = timed_region(step, args.steps, stream, torch)
    es = x.element_size()
    nbytes = float(rows) * n * 2 * es + rows * 4  # x read once, y written once, lse
    gbs = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": f"row softmax ({mode}) GB/s, {rows} rows of {n} ({w.name} score rows)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "fp16", "bf16": "bf16"}[w.dtype], "data": "synthetic",
        "config": {"workload": w.name, "rows": rows, "n": n, "path": args.path},
        "timing": timing_summary(ms, batches),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel_ms": round(ms, 5),
                     "algorithmic_units": "bytes per launch (x once, y once, lse)",
                     "algorithmic_per_launch": nbytes},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_qkv(args, w, torch, sdpa) -> int:
    """QKV projection of the workload's tokens (model width D = H*d, the
    weight [3*H*d, D]), alone or followed by the attention of the workload."""
    from scaled_dot_product_flashattention_amd.inputs import generate_qkv_proj

    B, S, H, d = w.B, w.Sq, w.H, w.d
    D = H * d
    dev = torch.device("cuda:0")
    t = generate_qkv_proj(B, S, D, H, d, w.dtype, seed=w.seed)
    x, wt = t["x"].to(dev), t["w"].to(dev)
    shape = sdpa.api.layout_shape(w.layout, B, H, S, d)
    if args.path == "qkv_attn_unfused" and w.layout not in ("bhsd", "bshd"):
        print("the unfused sequence is written for [B,H,S,d] and [B,S,H,d] only", file=sys.stderr)
        return 2
    qkv = tuple(torch.empty(shape, dtype=x.dtype, device=dev) for _ in range(3))
    o = torch.empty(shape, dtype=x.dtype, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    proj_flops = 2.0 * B * S * (3 * H * d) * D
    attn_flops = flops(w.replace(Sk=S, kv_len_range=None))
    akw = dict(scale=w.scale, causal=w.causal, layout=w.layout, out=o, lse=lse)
    if args.path == "qkv":
        step = lambda: sdpa.attn_qkv_proj(x, wt, H=H, d=d, layout=w.layout, out=qkv)  # noqa: E731
        fl = proj_flops
    elif args.path == "qkv_attn":
        def step():
            q, k, v = sdpa.attn_qkv_proj(x, wt, H=H, d=d, layout=w.layout, out=qkv)
            sdpa.attn_fwd(q, k, v, **akw)
        fl = proj_flops + attn_flops
    else:
        wq, wk, wv = (wt[i * H * d:(i + 1) * H * d] for i in range(3))

        def step():
            outs = []
            for wi in (wq, wk, wv):
                y = torch.matmul(x, wi.t()).view(B, S, H, d)
                outs.append(y.transpose(1, 2).contiguous() if w.layout == "bhsd" else y)
            sdpa.attn_fwd(*outs, **akw)
        fl = proj_flops + attn_flops
    prewarm(step, args.prewarm_s, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ms, batches = timed_region(step, args.steps, stream, torch)
    tflops = fl / (ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS_16, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_TFLOPS_16, 4), "traffic": None, "kernel_ms": round(ms, 5),
            "algorithmic_units": "FLOPs per step", "algorithmic_per_launch": fl}
    what = {"qkv": "QKV projection", "qkv_attn": "QKV projection + attention",
            "qkv_attn_unfused": "unfused projections + attention"}[args.path]
    line = {
        "metric": f"{what} TFLOP/s, tokens of {w.description}, D={D}",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"f16": "fp16", "bf16": "bf16"}[w.dtype], "data": "synthetic",
        "config": {"workload": w.name, "B": B, "S": S, "D": D, "H": H, "d": d, "layout": w.layout,
                   "causal": w.causal, "path": args.path, "flops_per_step": fl},
        "timing": timing_summary(ms, batches),
        "roofline": roof,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", default="medium_bf16")
    ap.add_argument("--path", default="fused",
                    choices=["fused", "naive", "splitk", "qkv", "qkv_attn", "qkv_attn_unfused",
                             "softmax_online", "softmax_three_pass"],
                    help="fused attention (default), the unfused baseline, the explicit "
                         "split-K path, the QKV projection alone, projection + attention, "
                         "the unfused sequence (three library matmuls and layout "
                         "copies, then attention), or the row softmax (online or "
                         "three-pass) over the workload's B*H*Sq score rows of Sk")
    ap.add_argument("--n-split", type=int, default=None)
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time graph replays (fused and "
                         "splitk paths)")
    ap.add_argument("--shape", default=None,
                    help="override the workload's B,H,Sq,Sk (e.g. 1,8,1,4096 for a small decode)")
    ap.add_argument("--layout", default=None,
                    help="override the workload's tensor layout: bhsd ([B,H,S,d]), bshd "
                         "([B,S,H,d]) or split:g ([B,H/g,S,g,d], heads in groups of g)")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm-s", type=float, default=0.2,
                    help="before the warmup steps, run steps for this many seconds so the "
                         "GPU reaches its sustained clock (0 to skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run 3 plain device copies of 256 MiB so a "
                         "counter profile of this run can scale its byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library is a "
              "single-GPU attention operator and has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import torch

    import scaled_dot_product_flashattention_amd as sdpa
    from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    w = WORKLOADS[args.config]
    relaid = args.layout is not None and args.layout != w.layout
    if relaid:
        w = w.replace(layout=args.layout)
    if args.shape:
        B_, H_, Sq_, Sk_ = (int(x) for x in args.shape.split(","))
        kv = None if w.kv_len_range is None else (min(w.kv_len_range[0], Sk_), Sk_)
        w = w.replace(B=B_, H=H_, Sq=Sq_, Sk=Sk_, kv_len_range=kv,
                      description=f"{w.name} at B{B_} H{H_} Sq{Sq_} Sk{Sk_}")
        relaid = True  # not the study's shape: no headline metric, no stored traffic
    if args.path.startswith("qkv"):
        return bench_qkv(args, w, torch, sdpa)
    if args.path.startswith("softmax"):
        return bench_softmax(args, w, torch, sdpa)
    t = generate(w)
    dev = torch.device("cuda:0")
    q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
    kv_len = None if t["kv_len"] is None else t["kv_len"].to(dev)
    B, H, Sq, Sk, d = w.B, w.H, w.Sq, w.Sk, w.d
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    kw = dict(scale=w.scale, causal=w.causal, layout=w.layout, kv_len=kv_len, out=o, lse=lse)
    tile = None
    if args.path == "fused":
        nbytes = sdpa.attn_fwd_workspace_size(B, H, Sq, Sk, d, q.dtype, w.causal)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        step = lambda: sdpa.attn_fwd(q, k, v, workspace=ws, **kw)  # noqa: E731
        n_split = sdpa.attn_fwd_plan(B, H, Sq, Sk, d, q.dtype, w.causal)
        if n_split == 1 or Sq > 1:  # the fused kernel, over all keys or over key ranges
            t_id = sdpa.attn_fwd_tile_choice(B, H, Sq, Sk, d, q.dtype, w.causal)
            tile = {"variant": t_id, **sdpa.attn_fwd_tile_info(d, q.dtype, t_id)}
    elif args.path == "splitk":
        n_split = args.n_split or sdpa.attn_fwd_plan(B, H, Sq, Sk, d, q.dtype, w.causal)
        ws = torch.empty(sdpa.attn_splitk_workspace_size(B, H, Sq, d, n_split), dtype=torch.uint8,
                         device=dev)
        step = lambda: sdpa.attn_fwd_splitk(q, k, v, n_split=n_split, workspace=ws, **kw)  # noqa: E731
    else:
        n_split = 1
        sc = torch.empty(sdpa.attn_naive_scratch_size(B, H, Sq, Sk, q.dtype), dtype=torch.uint8,
                         device=dev)
        step = lambda: sdpa.attn_fwd_naive(q, k, v, scratch=sc, **kw)  # noqa: E731

    prewarm_steps = prewarm(step, args.prewarm_s, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        if args.path == "naive":
            print("--graph covers the fused and splitk paths", file=sys.stderr)
            return 2
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        step = g.replay
        for _ in range(min(args.warmup, 50)):
            step()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t_wall = time.perf_counter()
    ms, batches = timed_region(step, args.steps, stream, torch)
    wall_ms = (time.perf_counter() - t_wall) * 1e3

    peak_bytes = torch.cuda.max_memory_allocated(dev)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    fl_nominal = flops(w)
    fl = algorithmic_flops(w, t["kv_len"])
    # the split-over-keys kernels run for one query per head
    splitk_kernels = args.path == "splitk" or (n_split > 1 and Sq == 1)
    # below the ridge (peak FLOP/s over peak bytes/s) the K/V stream bounds
    # the launch: few queries per head over many keys
    peak_fl = PEAK_TFLOPS_F32 if w.dtype == "f32" else PEAK_TFLOPS_16
    hbm_bound = splitk_kernels or fl / kv_bytes(w) < peak_fl * 1e3 / PEAK_HBM_GBS
    tflops = fl / (ms * 1e-3) / 1e12
    if hbm_bound:
        achieved = kv_bytes(w) / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
        what = "decode" if Sq == 1 else f"fwd ({args.path})"
        metric, value, unit = f"attention {what} HBM GB/s, {w.description}", achieved, "GB/s"
    else:
        peak = PEAK_TFLOPS_F32 if w.dtype == "f32" else PEAK_TFLOPS_16
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4)}
        mhz = None if relaid else stored_clock(args.config, args.path, "splitk" if splitk_kernels
                                                else args.path)
        if mhz:
            # the matrix peak scales with the shader clock (spec: 2400 MHz)
            peak_clk = peak * mhz / 2400.0
            roof["clock_mhz"] = round(mhz, 1)
            roof["clock_source"] = "GRBM_GUI_ACTIVE per dispatch over its duration, committed profile"
            roof["peak_at_measured_clock"] = round(peak_clk, 1)
            roof["frac_at_measured_clock"] = round(tflops / peak_clk, 4)
        if args.config == "medium_bf16" and args.path == "fused" and not relaid:
            metric = "fused attention fwd TFLOP/s and % bf16 MFMA peak, B1 H16 S4096 d64"
        else:
            metric = f"attention fwd TFLOP/s ({args.path}), {w.description}"
        value, unit = tflops, "TFLOP/s"
    kind = "splitk" if splitk_kernels else args.path
    roof["traffic"] = None if relaid else stored_traffic(args.config, args.path, kind)
    roof["kernel_ms"] = round(ms, 5)
    roof["algorithmic_units"] = ("bytes of K and V per launch" if hbm_bound else "FLOPs per launch")
    roof["algorithmic_per_launch"] = kv_bytes(w) if hbm_bound else fl

    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "fp16", "bf16": "bf16"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "B": B, "H": H, "Sq": Sq,
                   "Sk": Sk, "d": d, "layout": w.layout, "causal": w.causal, "path": args.path,
                   "graph": args.graph,
                   "n_split": n_split, "tile": tile, "flops_per_step": fl,
                   "flops_nominal": fl_nominal,
                   "flops_counted": "valid (query, key) pairs x 4d" if w.kv_len_range is not None
                   else "4*B*H*Sq*Sk*d" + (", halved (causal)" if w.causal else ""),
                   "wall_ms_timed_region": round(wall_ms, 2),
                   "peak_device_bytes": peak_bytes},
        "timing": timing_summary(ms, batches),
        "roofline": roof,
        "prewarm": {"seconds": args.prewarm_s, "steps": prewarm_steps},
    }
    if not args.skip_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, t, o, lse)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
