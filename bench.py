"""Benchmark of the WTConv layer on one MI355X: forward + backward (data and
parameter gradients) per step, on synthetic WTConvNeXt-shaped tensors.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stage1]

Prints ONE JSON line.  A step is one pass of the whole layer: wtconv_forward,
wtconv_backward_data and wtconv_backward_weight on one batch already resident
in device memory.  `value` is the achieved rate on the modeled minimum bytes
of a step (forward reads x and writes y, the data backward reads dy and
writes dx, the weight backward reads x and dy: 6 E e bytes for E elements of
e bytes).  Kernel durations are measured with HIP events on the stream the
library launches on.  The `roofline` object is for the dominant kernel of the
step; the `cpu_baseline` object times the CPU oracle on a bounded sample of
the same workload.  Other options:
    --cpu-sample N   images of the CPU-oracle sample (default: the whole batch; 0 disables it)
    --mall-flush     write a 512 MiB buffer between timed steps
    --all            also print one line per workload (stderr)
    --copy-calibration BYTES   only run a plain device copy (for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "WTConv fwd+bwd µs/layer and achieved HBM GB/s (% of peak), fp32/fp16, L=1–5"
HBM_PEAK_GBS = 8000.0
# fp32 FMA on the vector ALUs without packed instructions (the library is built
# with packed fp32 switched off): 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz
VALU_FP32_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
PACKED_FP32_PUBLISHED_TFLOPS = 157.3

CSRC = os.path.join(ROOT, "level_haar_wavelet_amd", "csrc")


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that a
    comment-only edit keeps the digest of code the counters were taken on."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """Digest of every kernel and launch source of the library (code only)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def conv_flops(wl) -> float:
    """Algorithmic FLOPs of one op: 2 k^2 (1 + S(L)) per element, S(L) = sum 4^(1-l)."""
    s = sum(4.0 ** (1 - l) for l in range(1, wl.levels + 1))
    return 2.0 * wl.k * wl.k * (1.0 + s) * wl.elems


def measured_traffic(kernel: str, digest: str, workload: str):
    """HBM bytes per launch of `kernel` (an op) on `workload` from the
    committed counter summary, if it was taken on the current kernel sources
    (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh).get(workload, {})
    except (OSError, ValueError, AttributeError):
        return None
    if d.get("source_digest") != digest:
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def workload_name(wl) -> str:
    return "%s %dx%dx%dx%d k=%d L=%d %s" % (wl.name, wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels,
                                           "fp32" if wl.dtype == "f32" else "fp16 storage")


_BUILTIN = {"f": "float", "d": "double", "i": "int", "j": "unsigned int", "b": "bool", "DF16_": "_Float16"}


def _demangle(name: str) -> str:
    """Function name and template arguments of an Itanium-mangled kernel name
    (the subset of the grammar kernel names here use: an optional nested name,
    builtin types and integer literals as template arguments); other names are
    returned unchanged."""
    if not name.startswith("_Z"):
        return name
    i, parts = 2, []

    def ident(i):
        j = i
        while j < len(name) and name[j].isdigit():
            j += 1
        n = int(name[i:j])
        return name[j:j + n], j + n

    try:
        if name[i] == "N":
            i += 1
            while name[i].isdigit():
                part, i = ident(i)
                parts.append(part)
        else:
            part, i = ident(i)
            parts.append(part)
        base = [p for p in parts if not p.startswith("_GLOBAL__N")][-1]
        if i >= len(name) or name[i] != "I":
            return base
        i += 1
        args = []
        while name[i] != "E":
            if name[i] == "L":
                j = name.index("E", i)
                t, v = name[i + 1], name[i + 2:j]
                args.append(("true" if v == "1" else "false") if t == "b" else v.replace("n", "-"))
                i = j + 1
            else:
                key = next(k for k in sorted(_BUILTIN, key=len, reverse=True) if name.startswith(k, i))
                args.append(_BUILTIN[key])
                i += len(key)
        return "%s<%s>" % (base, ", ".join(args))
    except (ValueError, IndexError, StopIteration):
        return name


def _short_kernel(name: str) -> str:
    """Kernel name without the return type and the parameter list, as profilers
    print it in any of its forms (plain, with its signature, or mangled)."""
    name = _demangle(name.strip())
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _counter_means(folder: str) -> dict:
    """Mean counter value per dispatch for each kernel, from the
    *counter_collection.csv files that `rocprofv3 --pmc` wrote under folder."""
    import csv
    import glob

    sums = {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                key = (_short_kernel(row["Kernel_Name"]), row["Counter_Name"])
                acc = sums.setdefault(key, {})
                acc[row["Dispatch_Id"]] = acc.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {key: sum(v.values()) / len(v) for key, v in sums.items()}


def traffic_summary(folder: str, workload: str, copy_bytes: int, outdir: str = None) -> dict:
    """Writes profiles/hbm_traffic.json and profiles/<workload>_hbm_traffic.md
    from four counter runs under folder: fetch/ and write/ (FETCH_SIZE and
    WRITE_SIZE of the bench), cfetch/ and cwrite/ (the same counters over a
    plain device copy of copy_bytes bytes, which scales KiB to bytes)."""
    from level_haar_wavelet_amd.synthetic import WORKLOADS

    outdir = outdir or os.path.join(ROOT, "profiles")
    wl = WORKLOADS[workload]
    fetch, write = _counter_means(os.path.join(folder, "fetch")), _counter_means(os.path.join(folder, "write"))
    cf, cw = _counter_means(os.path.join(folder, "cfetch")), _counter_means(os.path.join(folder, "cwrite"))
    copy_f = max(v for (k, c), v in cf.items() if c == "FETCH_SIZE")
    copy_w = max(v for (k, c), v in cw.items() if c == "WRITE_SIZE")
    ff, fw = copy_bytes / 1024.0 / copy_f, copy_bytes / 1024.0 / copy_w
    kernels = {}
    for (k, c), v in sorted(fetch.items()):
        if c == "FETCH_SIZE" and k.startswith(("wtconv_", "lowpass_")):
            kernels[k] = {"fetch_kib": v, "write_kib": write.get((k, "WRITE_SIZE"), 0.0),
                          "fetch_bytes": v * 1024.0 * ff, "write_bytes": write.get((k, "WRITE_SIZE"), 0.0) * 1024.0 * fw}
    whole = [k for k in kernels if k.startswith("wtconv_whole_kernel")]
    wgrad = [k for k in kernels if k.startswith("wtconv_wgrad_kernel")]
    fin = [k for k in kernels if k.startswith("wtconv_wgrad_finalize")]
    out = {"source_digest": source_digest(), "workload": workload_name(wl), "fetch_factor": ff, "write_factor": fw,
           "kernels": {k: {"fetch_bytes": v["fetch_bytes"], "write_bytes": v["write_bytes"]} for k, v in kernels.items()}}
    # per-op bytes where each op is one kernel launch (plus the reduction pass)
    if len(whole) == 1 and len(wgrad) == 1 and not any(k.startswith("lowpass_") for k in kernels):
        wb = kernels[whole[0]]["fetch_bytes"] + kernels[whole[0]]["write_bytes"]
        gb = sum(kernels[k]["fetch_bytes"] + kernels[k]["write_bytes"] for k in wgrad + fin)
        out["kernels"]["wtconv_forward"] = {"bytes_per_launch": wb}
        out["kernels"]["wtconv_backward_data"] = {"bytes_per_launch": wb}
        out["kernels"]["wtconv_backward_weight"] = {"bytes_per_launch": gb}
    # one entry per workload, merged into what the file already holds
    jpath = os.path.join(outdir, "hbm_traffic.json")
    try:
        with open(jpath) as fh:
            allw = json.load(fh)
        if "source_digest" in allw:  # a single-workload file of an earlier format
            allw = {}
    except (OSError, ValueError):
        allw = {}
    allw[out["workload"]] = out
    with open(jpath, "w") as fh:
        json.dump(allw, fh, indent=1)
    E, e = wl.elems, wl.ebytes
    bench = ("python3 bench.py --workload %s --steps 2 --warmup 1 --cpu-sample 0 --no-unfused --no-comparator"
             % workload)
    lines = ["# HBM traffic per launch: %s" % out["workload"], "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 counter runs, each scaled by what "
             "the same counter reads for a plain %d-byte device copy (`bench.py --copy-calibration %d`): "
             "FETCH_SIZE reads %.0f KiB for the copy's %.0f KiB (factor %.4f), WRITE_SIZE %.0f KiB (factor %.4f)."
             % (copy_bytes, copy_bytes, copy_f, copy_bytes / 1024.0, ff, copy_w, fw), "",
             "Commands (from the repository root; OUT is any output folder):", "",
             "    rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o fetch --output-format csv -- " + bench,
             "    rocprofv3 --pmc WRITE_SIZE -d OUT/write -o write --output-format csv -- " + bench,
             "    rocprofv3 --pmc FETCH_SIZE -d OUT/cfetch -o cfetch --output-format csv -- "
             "python3 bench.py --copy-calibration %d" % copy_bytes,
             "    rocprofv3 --pmc WRITE_SIZE -d OUT/cwrite -o cwrite --output-format csv -- "
             "python3 bench.py --copy-calibration %d" % copy_bytes,
             "    python3 bench.py --traffic-summary OUT --workload %s --copy-calibration %d" % (workload, copy_bytes),
             "", "| kernel | FETCH KiB | WRITE KiB | fetch bytes (scaled) | write bytes (scaled) |",
             "|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append("| `%s` | %.0f | %.0f | %.4g | %.4g |" % (k, v["fetch_kib"], v["write_kib"], v["fetch_bytes"],
                                                               v["write_bytes"]))
    lines += ["", "Counters per dispatch, averaged over all launches of a kernel (sizes mixed where one op "
              "launches it at several sizes).", "",
              "Modeled minimum per launch: forward or data backward %.4g bytes (read E e, write E e), weight "
              "backward %.4g bytes (read 2 E e)." % (2.0 * E * e, 2.0 * E * e), "",
              "Source digest of the kernels counted: `%s` (bench.py reports `traffic` only while the library "
              "sources still hash to it)." % out["source_digest"]]
    with open(os.path.join(outdir, "%s_hbm_traffic.md" % workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


def trace_summary(folder: str, workload: str, outdir: str = None) -> str:
    """Writes profiles/<workload>_kernel_trace.md from the *kernel_stats.csv of
    a `rocprofv3 --kernel-trace --stats` run under folder, with the bench line
    folder/bench.json (a plain run of the same build) if present."""
    import csv
    import glob

    from level_haar_wavelet_amd.synthetic import WORKLOADS

    outdir = outdir or os.path.join(ROOT, "profiles")
    wl = WORKLOADS[workload]
    name = workload_name(wl)
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True):
        with open(path, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    cmd = ("rocprofv3 --kernel-trace --stats -d OUT/kt -o kt --output-format csv -- python3 bench.py --workload %s "
           "--steps 5 --warmup 2 --cpu-sample 0 --no-unfused --no-comparator" % workload)
    lines = ["# Kernel durations: %s (MI355X)" % name, "", "Commands (from the repository root; OUT is any output "
             "folder):", "", "    " + cmd,
             "    python3 bench.py --workload %s > OUT/kt/bench.json" % workload,
             "    python3 bench.py --trace-summary OUT/kt --workload %s" % workload, "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f %% |" % (
            _short_kernel(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))
    lines += ["", "Before the 2 warm-up and 5 timed steps, bench.py runs the step for 0.5 s untimed (clock ramp), "
              "so the call counts are those of about half a second of steps.  A kernel launched at several sizes "
              "within one op (a tiled pass and the nested call on its level-1 low-pass map) is averaged over all "
              "its launches."]
    bj = os.path.join(folder, "bench.json")
    if os.path.exists(bj):
        with open(bj) as fh:
            line = [ln for ln in fh.read().splitlines() if ln.startswith("{")][-1]
        lines += ["", "bench.py line of the same build (`python3 bench.py --workload %s`):" % workload, "", "```",
                  line, "```"]
    path = os.path.join(outdir, "%s_kernel_trace.md" % workload)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def run_gpu(args, wl):
    import torch

    import level_haar_wavelet_amd as wt
    from level_haar_wavelet_amd import _native
    from level_haar_wavelet_amd.synthetic import make_inputs

    _native.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
    tdt = torch.float32 if wl.dtype == "f32" else torch.float16
    T = lambda a, dt=torch.float32: torch.from_numpy(a).to(dev, dtype=dt)
    x, dy = T(inp.x, tdt), T(inp.dy, tdt)
    w0, b0, s0, wl_, sl_ = T(inp.w_base), T(inp.bias), T(inp.s_base), T(inp.w_lvl), T(inp.s_lvl)
    y, dx = torch.empty_like(x), torch.empty_like(dy)
    ws_bytes = wt.wtconv_workspace_size((wl.n, wl.c, wl.h, wl.w), wl.k, wl.levels, 0 if wl.dtype == "f32" else 1,
                                        _native.OP_BWD_WEIGHT)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # forward / data-backward workspaces (planes too large for one workgroup keep
    # their level-1 low-pass map and deeper levels' term there), allocated once
    wsf = [torch.empty(max(wt.wtconv_workspace_size((wl.n, wl.c, wl.h, wl.w), wl.k, wl.levels,
                                                    0 if wl.dtype == "f32" else 1, op), 1),
                       dtype=torch.uint8, device=dev) for op in (_native.OP_FWD, _native.OP_BWD_DATA)]
    grads = (torch.empty_like(w0), torch.empty_like(b0), torch.empty_like(s0), torch.empty_like(wl_),
             torch.empty_like(sl_))
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.mall_flush else None
    stream = torch.cuda.current_stream()

    def step(ev=None, s=None):
        s = s or stream
        if ev:
            ev[0].record(s)
        wt.wtconv_forward(x, w0, b0, s0, wl_, sl_, y=y, stream=s, workspace=wsf[0])
        if ev:
            ev[1].record(s)
        wt.wtconv_backward_data(dy, w0, s0, wl_, sl_, dx=dx, stream=s, workspace=wsf[1])
        if ev:
            ev[2].record(s)
        wt.wtconv_backward_weight(x, dy, w0, b0, s0, wl_, sl_, workspace=ws, grads=grads, stream=s)
        if ev:
            ev[3].record(s)

    # the GPU raises its clocks only under sustained load: run the step for
    # about half a second (untimed) before the warm-up steps proper
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_s:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    if flush is None:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            step(evs[i])
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_total = start.elapsed_time(end)
    else:
        ms_total = 0.0
        t0 = time.perf_counter()
        for i in range(args.steps):
            flush.fill_(i & 255)
            torch.cuda.synchronize()
            step(evs[i])
            torch.cuda.synchronize()
            ms_total += evs[i][0].elapsed_time(evs[i][3])
        wall = time.perf_counter() - t0
    per = [[e[j].elapsed_time(e[j + 1]) * 1000.0 for j in range(3)] for e in evs]  # us per op and step
    med = [sorted(p[j] for p in per)[len(per) // 2] for j in range(3)]
    mean = [sum(p[j] for p in per) / len(per) for j in range(3)]
    out = {"ms_per_step": ms_total / args.steps, "us_ops": med, "us_ops_mean": mean, "wall_s": wall}
    if flush is None and args.graph:
        out["graph"] = graph_step_ms(torch, step, args.warmup, args.steps)
    return out


def graph_step_ms(torch, step, warmup, steps):
    """The same step captured once in a HIP graph (the library allocates
    nothing and only launches kernels on the stream it is given, so the three
    calls capture as they are) and replayed: K replays timed between two
    events, after W untimed ones.  Returns ms per step, or the error text if
    capture fails."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(s=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(s=torch.cuda.current_stream())
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        a.record(cur)
        for _ in range(steps):
            g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        return {"ms_per_step": a.elapsed_time(b) / steps}
    except RuntimeError as e:  # report, keep the eager measurement
        return {"error": str(e)[:200]}


def stream_copy_gbs(nbytes=1 << 30, reps=10):
    """Device-to-device copy rate on this GPU (bytes read + written per second,
    median of `reps` timed copies of `nbytes`): the practical HBM ceiling the
    achieved GB/s is read against."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del a, b
    torch.cuda.empty_cache()
    times.sort()
    return 2.0 * nbytes / times[len(times) // 2] / 1e9


def run_unfused(args, wl):
    """The same step on the unfused baseline (separate kernels, intermediates in
    HBM; wtconv_unfused_*), timed the same way, and the peak device memory of
    one forward + backward of each path (torch.cuda.max_memory_allocated above
    what the inputs, outputs and parameters already hold, workspaces included)."""
    import torch

    import level_haar_wavelet_amd as wt
    from level_haar_wavelet_amd import _native
    from level_haar_wavelet_amd import unfused as uf
    from level_haar_wavelet_amd.synthetic import make_inputs

    dev = torch.device("cuda:0")
    inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
    tdt = torch.float32 if wl.dtype == "f32" else torch.float16
    T = lambda a, dt=torch.float32: torch.from_numpy(a).to(dev, dtype=dt)
    x, dy = T(inp.x, tdt), T(inp.dy, tdt)
    w0, b0, s0, wl_, sl_ = T(inp.w_base), T(inp.bias), T(inp.s_base), T(inp.w_lvl), T(inp.s_lvl)
    y, dx = torch.empty_like(x), torch.empty_like(dy)
    grads = (torch.empty_like(w0), torch.empty_like(b0), torch.empty_like(s0), torch.empty_like(wl_),
             torch.empty_like(sl_))
    if wl.levels == 0:
        wl_ = sl_ = None
        grads = grads[:3] + (None, None)
    stream = torch.cuda.current_stream()

    def peak(fn):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    def fused_step():
        n = wt.wtconv_workspace_size((wl.n, wl.c, wl.h, wl.w), wl.k, wl.levels, 0 if wl.dtype == "f32" else 1,
                                     _native.OP_BWD_WEIGHT)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        wt.wtconv_forward(x, w0, b0, s0, wl_, sl_, y=y, stream=stream)
        wt.wtconv_backward_data(dy, w0, s0, wl_, sl_, dx=dx, stream=stream)
        wt.wtconv_backward_weight(x, dy, w0, b0, s0, wl_, sl_, workspace=ws, grads=grads, stream=stream)

    def unfused_step(ws=None):
        ws = uf.workspace(x, wl.k, wl.levels) if ws is None else ws
        uf.wtconv_unfused_forward(x, w0, b0, s0, wl_, sl_, ws, y=y, stream=stream)
        uf.wtconv_unfused_backward_data(dy, w0, s0, wl_, sl_, ws, dx=dx, stream=stream)
        uf.wtconv_unfused_backward_weight(x, dy, w0, b0, s0, wl_, sl_, ws, grads=grads, stream=stream)

    mem_fused, mem_unfused = peak(fused_step), peak(unfused_step)
    ws = uf.workspace(x, wl.k, wl.levels)
    ops = (lambda: uf.wtconv_unfused_forward(x, w0, b0, s0, wl_, sl_, ws, y=y, stream=stream),
           lambda: uf.wtconv_unfused_backward_data(dy, w0, s0, wl_, sl_, ws, dx=dx, stream=stream),
           lambda: uf.wtconv_unfused_backward_weight(x, dy, w0, b0, s0, wl_, sl_, ws, grads=grads, stream=stream))
    for _ in range(max(2, args.warmup // 2)):
        unfused_step(ws)
    steps = max(5, args.steps // 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record(stream)
        for j, op in enumerate(ops):
            op()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    per = [[e[j].elapsed_time(e[j + 1]) * 1000.0 for j in range(3)] for e in evs]
    med = [sorted(p[j] for p in per)[len(per) // 2] for j in range(3)]
    return {"us_ops": med, "steps": steps, "peak_mem_fused_bytes": int(mem_fused),
            "peak_mem_unfused_bytes": int(mem_unfused)}


def cpu_baseline(wl, images, min_seconds=2.0):
    """The CPU oracle (as it stands) on `images` images of the workload: one
    forward, data backward and weight backward, repeated until at least
    `min_seconds` have passed; the rate is the sample's own modeled bytes
    (6 E e per pass) over the mean time of a pass."""
    import oracle
    from level_haar_wavelet_amd.synthetic import make_inputs

    images = max(1, min(images, wl.n))
    inp = make_inputs(images, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
    threads = oracle.default_threads()
    try:
        threads = min(threads, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    args = (inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels)
    oracle.forward(inp.x[:1], *args, nthreads=1)  # load the library outside the timing
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp.x, *args, nthreads=threads)
        oracle.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels,
                             nthreads=threads)
        oracle.backward_weight(inp.x, inp.dy, *args, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 50:
            break
    per = dt / passes
    e = images * wl.c * wl.h * wl.w
    return {"value": round(6.0 * e * wl.ebytes / per / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d images (%dx%dx%dx%d), fwd + bwd_data + bwd_weight in fp64, %d passes, %.3f s/pass"
                      % (images, wl.n, images, wl.c, wl.h, wl.w, passes, per),
            "seconds_per_pass": round(per, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="stage1")
    ap.add_argument("--levels", type=int, default=None)
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--cpu-sample", type=int, default=64)
    ap.add_argument("--mall-flush", action="store_true")
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--trace-summary", default=None,
                    help="folder of a kernel-trace run: write the kernel-duration summary under profiles/ and exit")
    ap.add_argument("--traffic-summary", default=None,
                    help="folder of the four counter runs: write the HBM-traffic summaries under profiles/ and exit")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-baseline comparison")
    ap.add_argument("--no-comparator", action="store_true", help="skip the 7x7 depthwise comparator")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (reported as graph_ms_per_step)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU layer; more than one GPU is not supported in this build "
              "(the layer needs no collective for forward or data backward; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.workload))
        return

    if args.traffic_summary:
        print(json.dumps(traffic_summary(args.traffic_summary, args.workload, args.copy_calibration or (1 << 30)),
                         indent=1))
        return

    if args.copy_calibration:
        import torch

        a = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration}))
        return

    from level_haar_wavelet_amd.synthetic import WORKLOADS

    wl = WORKLOADS[args.workload]
    if args.levels is not None or args.dtype is not None:
        wl = wl.with_levels(args.levels if args.levels is not None else wl.levels, args.dtype)

    res = run_gpu(args, wl)
    E, e = wl.elems, wl.ebytes
    step_bytes = 6.0 * E * e
    # eager launches; with --graph the same step captured in a HIP graph and
    # replayed is reported next to it (it measured slower on MI355X, 223
    # against 205 us per step at stage1, so it does not set the value)
    graph = res.get("graph", {})
    ms = res["ms_per_step"]
    value = step_bytes / (ms * 1e-3) / 1e9
    us_f, us_b, us_w = res["us_ops"]
    flops = conv_flops(wl)
    # the roofline uses each op's average duration over the timed steps (the
    # statistic a kernel-trace summary reports)
    ops = dict(zip(("wtconv_forward", "wtconv_backward_data", "wtconv_backward_weight"), res["us_ops_mean"]))
    dominant = max(ops, key=ops.get)
    achieved = flops / (ops[dominant] * 1e-6) / 1e12
    digest = source_digest()
    traffic = measured_traffic(dominant, digest, workload_name(wl))
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ramp_s": args.ramp_s,
        "ms_per_step": round(ms, 4),
        "launch": "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": workload_name(wl),
                   "n": wl.n, "c": wl.c, "h": wl.h, "w": wl.w, "k": wl.k, "levels": wl.levels,
                   "parallelism": "single GPU"},
        "us_fwd": round(us_f, 2),
        "us_bwd_data": round(us_b, 2),
        "us_bwd_weight": round(us_w, 2),
        "us_fwd_bwd": round(us_f + us_b + us_w, 2),
        "us_per_op": "median over the timed steps (events around each call); means %s" % (
            ", ".join("%.2f" % v for v in res["us_ops_mean"])),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "stream_copy_GBs": round(stream_copy_gbs(), 1),
        "modeled_bytes_per_step": step_bytes,
        "mall_flush": bool(args.mall_flush),
        "graph_ms_per_step": round(graph["ms_per_step"], 4) if "ms_per_step" in graph else graph.get("error"),
        "roofline": {
            "bound": "alu",
            "kernel": dominant,
            "achieved": round(achieved, 3),
            "peak": round(VALU_FP32_PEAK_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": flops,
            "peak_published_packed_fp32": PACKED_FP32_PUBLISHED_TFLOPS,
            "source_digest": digest,
        },
    }
    if not args.no_unfused:
        u = run_unfused(args, wl)
        uf, ub, uw = u["us_ops"]
        line["unfused_baseline"] = {
            "what": "the same layer as separate kernels with every intermediate in HBM (wtconv_unfused_*), "
                    "timed the same way (medians over %d steps)" % u["steps"],
            "us_fwd": round(uf, 2), "us_bwd_data": round(ub, 2), "us_bwd_weight": round(uw, 2),
            "us_fwd_bwd": round(uf + ub + uw, 2),
            "speedup_fwd": round(uf / us_f, 3), "speedup_fwd_bwd": round((uf + ub + uw) / (us_f + us_b + us_w), 3),
            "peak_mem_fused_MB": round(u["peak_mem_fused_bytes"] / 2 ** 20, 1),
            "peak_mem_unfused_MB": round(u["peak_mem_unfused_bytes"] / 2 ** 20, 1),
        }
    if not args.no_comparator:
        # the same shape through a plain 7 x 7 depthwise convolution with bias
        # and scale (the library at L = 0, k = 7): the layer the method's
        # accuracy and cost are compared with
        import dataclasses

        dw = dataclasses.replace(wl, name=wl.name + "-dw7x7", k=7, levels=0)
        r7 = run_gpu(args, dw)
        f7, b7, w7 = r7["us_ops"]
        line["dw7x7_comparator"] = {
            "what": "7x7 depthwise conv (+bias, scale) on the same tensors, same timing",
            "us_fwd": round(f7, 2), "us_bwd_data": round(b7, 2), "us_bwd_weight": round(w7, 2),
            "us_fwd_bwd": round(f7 + b7 + w7, 2),
            "flops_per_element": 2 * 49, "wtconv_flops_per_element": round(conv_flops(wl) / wl.elems, 2),
            "wtconv_over_dw7x7_fwd": round(us_f / f7, 3),
            "wtconv_over_dw7x7_fwd_bwd": round((us_f + us_b + us_w) / (f7 + b7 + w7), 3),
        }
    if args.cpu_sample > 0:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    print(json.dumps(line), flush=True)

    if args.all:
        from level_haar_wavelet_amd.synthetic import sweep_workloads

        for w2 in [WORKLOADS["stage2"]] + sweep_workloads() + [WORKLOADS["large"]]:
            r2 = run_gpu(args, w2)
            ms2 = r2["ms_per_step"]
            v2 = 6.0 * w2.elems * w2.ebytes / (ms2 * 1e-3) / 1e9
            print(json.dumps({"workload": w2.name, "levels": w2.levels, "dtype": w2.dtype,
                              "us_fwd": round(r2["us_ops"][0], 2), "us_bwd_data": round(r2["us_ops"][1], 2),
                              "us_bwd_weight": round(r2["us_ops"][2], 2), "ms_per_step": round(ms2, 4),
                              "GB/s": round(v2, 1), "hbm_frac": round(v2 / HBM_PEAK_GBS, 4)}), file=sys.stderr,
                  flush=True)


if __name__ == "__main__":
    main()
