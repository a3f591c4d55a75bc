"""Benchmark of the WTConv layer on one MI355X: forward + backward (data and
parameter gradients) on synthetic WTConvNeXt-shaped tensors.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sweep]

Prints ONE JSON line.  The default workload is the level sweep the metric is
quoted on: N=32, C=128, H=W=128, k=5, L = 1..5, each in fp32 and in fp16
storage (fp32 arithmetic), ten points.  A step is one pass of the whole layer
(wtconv_forward, wtconv_backward_data, wtconv_backward_weight) at every point,
on batches already resident in device memory.  `value` is the achieved rate on
the modeled minimum bytes: the ten points' 6 E e bytes each (forward reads x
and writes y, the data backward reads dy and writes dx, the weight backward
reads x and dy; E elements of e bytes), summed, over the step time.  Per point
the line gives the median microseconds of every op, the step, its GB/s and its
fraction of the 8 TB/s HBM peak.  Op durations are HIP events recorded around
each call on the stream the library launches on.  The `roofline` object is
for the dominant op (the longest mean op duration of any point); `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.

Other modes:
    --workload stage1|stage2|large|tiny   one workload (with --levels/--dtype for one sweep point)
    --counter-op fwd|bwd_data|bwd_weight|unfused_fwd  only that op, --reps times after one warm call
                    (the program profiled by the counter runs)
    --traffic-summary OUT   HBM bytes per op from counter runs under OUT (see traffic_summary)
    --valu-summary OUT      VALU / LDS counter summary from counter runs under OUT
    --trace-summary OUT     kernel-duration summary from a kernel-trace run under OUT
    --copy-calibration BYTES   only a plain device copy of BYTES (counter scaling)
    --mall-flush            write a 512 MiB buffer between timed steps
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "WTConv fwd+bwd µs/layer and achieved HBM GB/s (% of peak), fp32/fp16, L=1–5"
# MI355X published peaks: HBM3E 8 TB/s; fp32 vector 157.3 TFLOP/s, i.e. 256 CUs x
# 2.4 GHz x 256 FLOP per clock per CU, which counts packed fp32 FMAs.  The
# library is built with packed fp32 switched off, so its reachable fp32 vector
# rate is half of that (256 x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz = 78.6
# TFLOP/s), reported next to the published roof.
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3
FP32_NONPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
RIDGE_FLOP_PER_BYTE = FP32_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

CSRC = os.path.join(ROOT, "level_haar_wavelet_amd", "csrc")
OPS = ("wtconv_forward", "wtconv_backward_data", "wtconv_backward_weight")
OP_KEYS = {"fwd": "wtconv_forward", "bwd_data": "wtconv_backward_data", "bwd_weight": "wtconv_backward_weight",
           "unfused_fwd": "wtconv_unfused_forward"}


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


def level_sum(levels: int) -> float:
    """S(L) = sum over l = 1..L of 4^(1-l): the level maps' share of the pixels."""
    return sum(4.0 ** (1 - l) for l in range(1, levels + 1))


def conv_flops(wl) -> float:
    """Algorithmic FLOPs of one op: 2 k^2 (1 + S(L)) per element."""
    return 2.0 * wl.k * wl.k * (1.0 + level_sum(wl.levels)) * wl.elems


def op_bytes(wl) -> float:
    """Algorithmic bytes of one op: two activation tensors (read x and write y,
    read dy and write dx, or read x and dy)."""
    return 2.0 * wl.elems * wl.ebytes


def unfused_forward_elements(wl) -> float:
    """Element moves of the unfused forward: (7 + 10.75 S(L)) E (per level a
    Haar analysis, a convolution and a scale pass, the low-pass add, the band
    concatenation and the synthesis at 4^(1-l) of the size, plus the base
    convolution, its scale and the final add); 17.75 E at L = 1 and 21.32 E at
    L = 5, the two ends of the count the pages give for the reference layer."""
    return (7.0 + 10.75 * level_sum(wl.levels)) * wl.elems


def workload_name(wl) -> str:
    return "%s %dx%dx%dx%d k=%d L=%d %s" % (wl.name, wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels,
                                           "fp32" if wl.dtype == "f32" else "fp16 storage")


def measured_traffic(op: str, digest: str, workload: str):
    """HBM bytes per call of `op` (all its kernel launches) on `workload` from
    the committed counter summary, if it was taken on the current kernel
    sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh).get(workload, {})
    except (OSError, ValueError, AttributeError):
        return None
    if d.get("source_digest") != digest:
        return None
    k = d.get("ops", {}).get(op)
    return None if k is None else k.get("bytes_per_launch")


def roofline(wl, op: str, mean_us: float, digest: str) -> dict:
    """Roofline of one op at one workload: the bound is the published roof its
    arithmetic intensity meets first (HBM below the ridge of 157.3 TFLOP/s over
    8 TB/s = 19.7 FLOP/B, the fp32 vector ALUs above it); `achieved` is the
    algorithmic bytes (or FLOPs) of one call over its mean duration."""
    flops, nbytes = conv_flops(wl), op_bytes(wl)
    t = mean_us * 1e-6
    intensity = flops / nbytes
    tflops, gbs = flops / t / 1e12, nbytes / t / 1e9
    if intensity < RIDGE_FLOP_PER_BYTE:
        out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        out = {"bound": "alu", "achieved": round(tflops, 3), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": round(tflops / FP32_PEAK_TFLOPS, 4)}
    out.update({
        "traffic": measured_traffic(op, digest, workload_name(wl)),
        "kernel": op, "workload": workload_name(wl), "mean_us": round(mean_us, 2),
        "bytes_per_launch": nbytes, "flops_per_launch": flops, "intensity_flop_per_byte": round(intensity, 2),
        "achieved_GBs": round(gbs, 1), "achieved_TFLOPs": round(tflops, 3),
        "nonpacked_fp32_peak_TFLOPs": round(FP32_NONPACKED_TFLOPS, 1),
        "nonpacked_fp32_frac": round(tflops / FP32_NONPACKED_TFLOPS, 4),
        "source_digest": digest,
    })
    return out


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
    name = name.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _counter_rows(folder: str):
    """(dispatch id, kernel, counter, value) of every *counter_collection.csv
    that `rocprofv3 --pmc` wrote under folder (values of one dispatch summed
    over the rows it spans)."""
    import csv
    import glob

    acc = {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                key = (int(row["Dispatch_Id"]), _short_kernel(row["Kernel_Name"]), row["Counter_Name"])
                acc[key] = acc.get(key, 0.0) + float(row["Counter_Value"])
    return [(d, k, c, v) for (d, k, c), v in sorted(acc.items())]


def _library_kernel(k: str) -> bool:
    return not k.startswith("__amd_")  # every kernel but the runtime's own copies


def traffic_summary(folder: str, wl, reps: int, copy_bytes: int, outdir: str = None) -> dict:
    """HBM bytes per op from counter runs of `bench.py --counter-op OP --reps
    reps` (reps + 1 calls of the op and nothing else): OUT/<op>_fetch and
    OUT/<op>_write (FETCH_SIZE and WRITE_SIZE, KiB per dispatch) for each op
    run, and OUT/cfetch, OUT/cwrite (the same counters over a plain device copy
    of copy_bytes bytes, which scale KiB to bytes).  An op's bytes are its
    kernels' scaled counters summed over all dispatches, divided by the calls.
    Writes profiles/hbm_traffic.json (one entry per workload, merged) and a
    markdown summary named for the workload."""
    outdir = outdir or os.path.join(ROOT, "profiles")
    cf = [v for _, _, c, v in _counter_rows(os.path.join(folder, "cfetch")) if c == "FETCH_SIZE"]
    cw = [v for _, _, c, v in _counter_rows(os.path.join(folder, "cwrite")) if c == "WRITE_SIZE"]
    copy_f, copy_w = max(cf), max(cw)
    ff, fw = copy_bytes / 1024.0 / copy_f, copy_bytes / 1024.0 / copy_w
    calls = reps + 1
    name = workload_name(wl)
    ops = {}
    for key, op in OP_KEYS.items():
        fr = _counter_rows(os.path.join(folder, key + "_fetch"))
        wr = _counter_rows(os.path.join(folder, key + "_write"))
        if not fr or not wr:
            continue
        kern = {}
        for _, k, c, v in fr:
            if c == "FETCH_SIZE" and _library_kernel(k):
                e = kern.setdefault(k, {"dispatches": 0, "fetch_bytes": 0.0, "write_bytes": 0.0})
                e["dispatches"] += 1
                e["fetch_bytes"] += v * 1024.0 * ff / calls
        for _, k, c, v in wr:
            if c == "WRITE_SIZE" and _library_kernel(k):
                e = kern.setdefault(k, {"dispatches": 0, "fetch_bytes": 0.0, "write_bytes": 0.0})
                e["write_bytes"] += v * 1024.0 * fw / calls
        for e in kern.values():
            e["dispatches"] = e["dispatches"] / calls
        f = sum(e["fetch_bytes"] for e in kern.values())
        w = sum(e["write_bytes"] for e in kern.values())
        model = unfused_forward_elements(wl) * wl.ebytes if key == "unfused_fwd" else op_bytes(wl)
        ops[op] = {"fetch_bytes": f, "write_bytes": w, "bytes_per_launch": f + w, "modeled_bytes": model,
                   "ratio_to_model": (f + w) / model, "kernels": kern}
    out = {"source_digest": source_digest(), "workload": name, "fetch_factor": ff, "write_factor": fw,
           "calls_per_run": calls, "ops": ops}
    jpath = os.path.join(outdir, "hbm_traffic.json")
    try:
        with open(jpath) as fh:
            allw = json.load(fh)
        if "source_digest" in allw:  # a single-workload file of an earlier format
            allw = {}
    except (OSError, ValueError):
        allw = {}
    allw[name] = out
    with open(jpath, "w") as fh:
        json.dump(allw, fh, indent=1)
    sel = "--workload %s%s" % (wl.name, point_args(wl))
    lines = ["# HBM traffic per op: %s" % name, "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 counter runs per op, each scaled by "
             "what the same counter reads for a plain %d-byte device copy (`bench.py --copy-calibration %d`): "
             "FETCH_SIZE reads %.0f KiB for the copy's %.0f KiB (factor %.4f), WRITE_SIZE %.0f KiB (factor %.4f). "
             "Each run calls the op %d times and nothing else; an op's bytes are the sum over its kernels' "
             "dispatches divided by the calls." % (copy_bytes, copy_bytes, copy_f, copy_bytes / 1024.0, ff, copy_w,
                                                   fw, calls), "",
             "Commands (from the repository root; OUT is any output folder; OP is fwd, bwd_data, bwd_weight "
             "or unfused_fwd):", "",
             "    rocprofv3 --pmc FETCH_SIZE -d OUT/OP_fetch -o f --output-format csv -- "
             "python3 bench.py %s --counter-op OP --reps %d" % (sel, reps),
             "    rocprofv3 --pmc WRITE_SIZE -d OUT/OP_write -o w --output-format csv -- "
             "python3 bench.py %s --counter-op OP --reps %d" % (sel, reps),
             "    rocprofv3 --pmc FETCH_SIZE -d OUT/cfetch -o f --output-format csv -- "
             "python3 bench.py --copy-calibration %d" % copy_bytes,
             "    rocprofv3 --pmc WRITE_SIZE -d OUT/cwrite -o w --output-format csv -- "
             "python3 bench.py --copy-calibration %d" % copy_bytes,
             "    python3 bench.py --traffic-summary OUT %s --reps %d --copy-calibration %d" % (sel, reps, copy_bytes),
             "", "| op | kernel | launches per call | fetch bytes | write bytes |", "|---|---|---|---|---|"]
    for op, d in ops.items():
        for k, e in d["kernels"].items():
            lines.append("| %s | `%s` | %.2f | %.4g | %.4g |" % (op, k, e["dispatches"], e["fetch_bytes"],
                                                                  e["write_bytes"]))
    lines += ["", "| op | fetch bytes | write bytes | total | modeled | ratio |", "|---|---|---|---|---|---|"]
    for op, d in ops.items():
        lines.append("| %s | %.4g | %.4g | %.4g | %.4g | %.3f |" % (op, d["fetch_bytes"], d["write_bytes"],
                                                                      d["bytes_per_launch"], d["modeled_bytes"],
                                                                      d["ratio_to_model"]))
    lines += ["", "Modeled bytes: 2 E e per fused op (E = %d elements of %d bytes); for the unfused forward "
              "(7 + 10.75 S(L)) E e, S(L) = sum 4^(1-l)." % (wl.elems, wl.ebytes), "",
              "Source digest of the kernels counted: `%s` (bench.py reports `traffic` only while the library "
              "sources still hash to it)." % out["source_digest"]]
    with open(os.path.join(outdir, "%s_hbm_traffic.md" % file_stem(wl)), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


VALU_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VALU_FMA_F32", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS",
                 "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")
XCDS = 8        # MI355X: GRBM_GUI_ACTIVE is summed over its eight XCDs
SIMDS = 1024    # 256 compute units x 4 SIMDs


def valu_summary(folder: str, wl, reps: int, outdir: str = None) -> str:
    """VALU and LDS counters per op from `rocprofv3 --pmc <VALU_COUNTERS>` runs
    of `bench.py --counter-op OP` under OUT/<op>_valu, per kernel and dispatch
    averaged over its dispatches: instructions per wave, the FMA share of the
    VALU instructions, VALU busy = SQ_ACTIVE_INST_VALU x 4 / (1024 SIMDs x
    GRBM_GUI_ACTIVE per XCD) (the fraction of the SIMDs' cycles spent issuing
    VALU instructions), and LDS bank-conflict cycles per LDS-active cycle."""
    outdir = outdir or os.path.join(ROOT, "profiles")
    sel = "--workload %s%s" % (wl.name, point_args(wl))
    lines = ["# VALU and LDS counters per op: %s (MI355X)" % workload_name(wl), "",
             "Commands (from the repository root; OUT is any output folder; OP is fwd, bwd_data or bwd_weight):", "",
             "    rocprofv3 --pmc %s -d OUT/OP_valu -o v --output-format csv -- python3 bench.py %s "
             "--counter-op OP --reps %d" % (" ".join(VALU_COUNTERS), sel, reps),
             "    python3 bench.py --valu-summary OUT %s --reps %d" % (sel, reps), "",
             "Per dispatch, averaged over the dispatches of a kernel.  VALU busy = SQ_ACTIVE_INST_VALU x 4 / "
             "(1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); FMA share = SQ_INSTS_VALU_FMA_F32 / SQ_INSTS_VALU; "
             "conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS; us = GRBM_GUI_ACTIVE / 8 / 2.4 GHz (the "
             "busy time at the published clock, for orientation).", "",
             "| op | kernel | dispatches | waves | VALU instr / wave | FMA share | LDS instr / wave | VALU busy | "
             "LDS conflict | us |", "|---|---|---|---|---|---|---|---|---|---|"]
    for key in ("fwd", "bwd_data", "bwd_weight"):
        rows = _counter_rows(os.path.join(folder, key + "_valu"))
        per = {}
        for d, k, c, v in rows:
            if _library_kernel(k):
                per.setdefault(k, {}).setdefault(d, {})[c] = v
        for k, disp in per.items():
            n = len(disp)
            mean = {c: sum(x.get(c, 0.0) for x in disp.values()) / n for c in VALU_COUNTERS}
            waves = max(mean["SQ_WAVES"], 1.0)
            gui = max(mean["GRBM_GUI_ACTIVE"] / XCDS, 1.0)
            busy = mean["SQ_ACTIVE_INST_VALU"] * 4.0 / (SIMDS * gui)
            fma = mean["SQ_INSTS_VALU_FMA_F32"] / max(mean["SQ_INSTS_VALU"], 1.0)
            conf = mean["SQ_LDS_BANK_CONFLICT"] / max(mean["SQ_ACTIVE_INST_LDS"], 1.0)
            lines.append("| %s | `%s` | %.2f | %.0f | %.0f | %.3f | %.0f | %.3f | %.3f | %.1f |" % (
                OP_KEYS[key], k, n / (reps + 1), waves, mean["SQ_INSTS_VALU"] / waves, fma,
                mean["SQ_INSTS_LDS"] / waves, busy, conf, gui / 2.4e3))
    lines += ["", "dispatches: launches of the kernel per call of the op.", "",
              "Source digest of the kernels counted: `%s`." % source_digest()]
    path = os.path.join(outdir, "%s_valu_lds.md" % file_stem(wl))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def point_args(wl) -> str:
    from level_haar_wavelet_amd.synthetic import WORKLOADS

    base = WORKLOADS[wl.name]
    return "" if (base.levels, base.dtype) == (wl.levels, wl.dtype) else " --levels %d --dtype %s" % (wl.levels,
                                                                                                     wl.dtype)


def file_stem(wl) -> str:
    """File name stem of a workload's summaries: its name, and for the level
    sweep the level and storage type."""
    return wl.name if wl.name != "sweep" else "sweep_L%d_%s" % (wl.levels, wl.dtype)


def trace_summary(folder: str, wl, outdir: str = None) -> str:
    """Writes profiles/<workload>_kernel_trace.md from the *kernel_stats.csv of
    a `rocprofv3 --kernel-trace --stats` run under folder, with the bench line
    folder/bench.json (a plain run of the same build) if present."""
    import csv
    import glob

    outdir = outdir or os.path.join(ROOT, "profiles")
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True):
        with open(path, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    sel = "--workload %s%s" % (wl.name, point_args(wl))
    cmd = ("rocprofv3 --kernel-trace --stats -d OUT/kt -o kt --output-format csv -- python3 bench.py %s "
           "--steps 5 --warmup 2 --cpu-sample 0 --no-unfused --no-comparator" % sel)
    lines = ["# Kernel durations: %s (MI355X)" % workload_name(wl), "",
             "Commands (from the repository root; OUT is any output folder):", "", "    " + cmd,
             "    python3 bench.py %s --cpu-sample 0 --no-unfused --no-comparator > OUT/kt/bench.json" % sel,
             "    python3 bench.py --trace-summary OUT/kt %s" % sel, "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f %% |" % (
            _short_kernel(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines += ["", "Before the 2 warm-up and 5 timed steps, bench.py runs the step for 0.5 s untimed (clock ramp), "
              "so the call counts are those of about half a second of steps.  A kernel launched at several sizes "
              "within one op is averaged over all its launches."]
    bj = os.path.join(folder, "bench.json")
    if os.path.exists(bj):
        with open(bj) as fh:
            line = [ln for ln in fh.read().splitlines() if ln.startswith("{")][-1]
        lines += ["", "bench.py line of the same build:", "", "```", line, "```"]
    path = os.path.join(outdir, "%s_kernel_trace.md" % file_stem(wl))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


# ---- GPU runs ----------------------------------------------------------------


class Point:
    """One workload point resident on the GPU: inputs, outputs, parameters,
    gradient buffers and the three ops' workspaces."""

    def __init__(self, wl, x, dy, params):
        import torch

        import level_haar_wavelet_amd as wt
        from level_haar_wavelet_amd import _native

        self.wl = wl
        dev = x.device
        self.x, self.dy = x, dy
        self.y, self.dx = torch.empty_like(x), torch.empty_like(dy)
        self.w0, self.b0, self.s0, self.wl_, self.sl_ = params
        dt = 0 if wl.dtype == "f32" else 1
        shape = (wl.n, wl.c, wl.h, wl.w)
        self.ws = [torch.empty(max(wt.wtconv_workspace_size(shape, wl.k, wl.levels, dt, op), 1), dtype=torch.uint8,
                               device=dev) for op in (_native.OP_FWD, _native.OP_BWD_DATA, _native.OP_BWD_WEIGHT)]
        self.grads = tuple(torch.empty_like(t) if t is not None else None for t in params)

    def ops(self, stream):
        import level_haar_wavelet_amd as wt

        return (lambda: wt.wtconv_forward(self.x, self.w0, self.b0, self.s0, self.wl_, self.sl_, y=self.y,
                                          stream=stream, workspace=self.ws[0]),
                lambda: wt.wtconv_backward_data(self.dy, self.w0, self.s0, self.wl_, self.sl_, dx=self.dx,
                                                stream=stream, workspace=self.ws[1]),
                lambda: wt.wtconv_backward_weight(self.x, self.dy, self.w0, self.b0, self.s0, self.wl_, self.sl_,
                                                  workspace=self.ws[2], grads=self.grads, stream=stream))


def make_points(wls):
    """Device-resident points for a list of workloads.  Sweep points share
    their activations: the inputs are drawn in the order x, dy, base
    parameters, then level by level, so every level count of one seed has the
    same x and dy and its parameters are a prefix of the deepest one's."""
    import numpy as np
    import torch

    from level_haar_wavelet_amd.synthetic import make_inputs

    dev = torch.device("cuda:0")
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dtype=dt)
    cache, points = {}, []
    for wl in wls:
        key = (wl.name, wl.n, wl.c, wl.h, wl.w, wl.k, wl.seed)
        if key not in cache:
            deepest = max(w.levels for w in wls if (w.name, w.n, w.c, w.h, w.w, w.k, w.seed) == key)
            inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, deepest, dtype="f32", seed=wl.seed)
            cache[key] = {"inp": inp, "act": {}}
        ent = cache[key]
        inp = ent["inp"]
        if wl.dtype not in ent["act"]:
            tdt = torch.float32 if wl.dtype == "f32" else torch.float16
            # fp16 storage: the fp32 draws rounded to fp16, as the recipe does
            ent["act"][wl.dtype] = (T(inp.x, tdt), T(inp.dy, tdt))
        x, dy = ent["act"][wl.dtype]
        L = wl.levels
        params = (T(inp.w_base), T(inp.bias), T(inp.s_base), T(inp.w_lvl[:L]) if L else None,
                  T(inp.s_lvl[:L]) if L else None)
        points.append(Point(wl, x, dy, params))
    for ent in cache.values():
        ent["inp"].x = ent["inp"].dy = None
    return points


def time_points(args, points):
    """Times the step -- the three ops at every point -- K times after the
    clock ramp and W warm-up steps.  Returns the step time and, per point and
    op, the median and mean of the event-timed durations."""
    import torch

    stream = torch.cuda.current_stream()
    ops = [p.ops(stream) for p in points]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0") if args.mall_flush else None

    def step(ev=None):
        for i, po in enumerate(ops):
            if ev:
                ev[i][0].record(stream)
            for j, op in enumerate(po):
                op()
                if ev:
                    ev[i][j + 1].record(stream)

    # the GPU raises its clocks only under sustained load: run the step for
    # about half a second (untimed) before the warm-up steps proper
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_s:
        for _ in range(3):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in points] for _ in range(args.steps)]
    if flush is None:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(args.steps):
            step(evs[s])
        end.record(stream)
        torch.cuda.synchronize()
        ms_total = start.elapsed_time(end)
    else:
        ms_total = 0.0
        for s in range(args.steps):
            flush.fill_(s & 255)
            torch.cuda.synchronize()
            step(evs[s])
            torch.cuda.synchronize()
            ms_total += evs[s][0][0].elapsed_time(evs[s][-1][3])
    res = []
    for i in range(len(points)):
        per = [[evs[s][i][j].elapsed_time(evs[s][i][j + 1]) * 1000.0 for j in range(3)] for s in range(args.steps)]
        med = [sorted(p[j] for p in per)[len(per) // 2] for j in range(3)]
        mean = [sum(p[j] for p in per) / len(per) for j in range(3)]
        step_us = sorted(sum(p) for p in per)[len(per) // 2]
        res.append({"us_ops": med, "us_ops_mean": mean, "us_step": step_us})
    return ms_total / args.steps, res


def time_backward(args, wl, reps=None, fused=True):
    """Median microseconds of wtconv_backward (dx and every gradient in one
    call; fused: the single pass over x and dy, WTCONV_FUSED_BWD=1) at one
    workload, timed like the step's ops, after the same clock ramp."""
    old = os.environ.get("WTCONV_FUSED_BWD")
    os.environ["WTCONV_FUSED_BWD"] = "1" if fused else "0"
    try:
        return _time_backward(args, wl, reps)
    finally:
        if old is None:
            os.environ.pop("WTCONV_FUSED_BWD", None)
        else:
            os.environ["WTCONV_FUSED_BWD"] = old


def _time_backward(args, wl, reps):
    import torch

    import level_haar_wavelet_amd as wt
    from level_haar_wavelet_amd import _native

    p = make_points([wl])[0]
    stream = torch.cuda.current_stream()
    dt = 0 if wl.dtype == "f32" else 1
    n = wt.wtconv_workspace_size((wl.n, wl.c, wl.h, wl.w), wl.k, wl.levels, dt, _native.OP_BWD)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda:0")
    op = lambda: wt.wtconv_backward(p.x, p.dy, p.w0, p.b0, p.s0, p.wl_, p.sl_, dx=p.dx, grads=p.grads,
                                    workspace=ws, stream=stream)
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_s:
        for _ in range(3):
            op()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        op()
    reps = reps or args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        op()
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)
    return ts[len(ts) // 2]


def make_block(c, dtype):
    """A synthetic WTConvNeXt-style block around the layer: LayerNorm over the
    channels, then a pointwise MLP (C -> 4C, GELU, 4C -> C), added back to the
    block's input (random init, seed 0)."""
    import torch

    torch.manual_seed(0)
    mods = torch.nn.ModuleDict({"norm": torch.nn.LayerNorm(c), "fc1": torch.nn.Linear(c, 4 * c),
                                "fc2": torch.nn.Linear(4 * c, c)}).cuda()
    return mods.to(dtype)


def block_step(mods, layer, x, params):
    """One training step of the block (forward, loss, backward)."""
    import torch

    h = layer(x, *params)
    t = h.permute(0, 2, 3, 1)
    t = mods["fc2"](torch.nn.functional.gelu(mods["fc1"](mods["norm"](t))))
    out = x + t.permute(0, 3, 1, 2)
    out.float().square().mean().backward()


def block_memory(wl) -> dict:
    """Peak device memory of one training step of the synthetic block with the
    fused layer (it saves only its input) and with the unfused baseline (it
    keeps its intermediates for the backward): torch.cuda.max_memory_allocated
    above what the block's input and parameters already hold."""
    import torch

    from level_haar_wavelet_amd.module import WTConvFunction
    from level_haar_wavelet_amd.synthetic import make_inputs
    from level_haar_wavelet_amd.unfused import UnfusedWTConvFunction

    tdt = torch.float32 if wl.dtype == "f32" else torch.float16
    inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp.x).to(dev, dtype=tdt).requires_grad_(True)
    params = [torch.from_numpy(a).to(dev).requires_grad_(True)
              for a in (inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl)]
    mods = make_block(wl.c, tdt)
    out = {}
    for name, layer in (("fused", WTConvFunction.apply), ("unfused", UnfusedWTConvFunction.apply)):
        block_step(mods, layer, x, params)  # warm (library plans, cuBLAS-like handles)
        for t in [x] + params + list(mods.parameters()):
            t.grad = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        block_step(mods, layer, x, params)
        torch.cuda.synchronize()
        out[name] = torch.cuda.max_memory_allocated() - base
        for t in [x] + params + list(mods.parameters()):
            t.grad = None
    return {"what": "one training step (forward, loss, backward) of a synthetic WTConvNeXt-style block: the layer, "
                    "LayerNorm over the channels, a pointwise MLP C -> 4C -> C with GELU, residual add; peak "
                    "device memory above the input and parameters",
            "workload": workload_name(wl), "peak_MB_fused": round(out["fused"] / 2 ** 20, 1),
            "peak_MB_unfused": round(out["unfused"] / 2 ** 20, 1),
            "unfused_over_fused": round(out["unfused"] / max(out["fused"], 1), 3)}


def point_record(wl, r) -> dict:
    f, b, w = r["us_ops"]
    gbs = 6.0 * wl.elems * wl.ebytes / (r["us_step"] * 1e-6) / 1e9
    return {"levels": wl.levels, "dtype": wl.dtype, "us_fwd": round(f, 2), "us_bwd_data": round(b, 2),
            "us_bwd_weight": round(w, 2), "us_fwd_bwd": round(r["us_step"], 2), "GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "fwd_GBs": round(op_bytes(wl) / (f * 1e-6) / 1e9, 1),
            "fwd_hbm_frac": round(op_bytes(wl) / (f * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


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

    p = make_points([wl])[0]
    x, dy, y, dx = p.x, p.dy, p.y, p.dx
    w0, b0, s0, wl_, sl_ = p.w0, p.b0, p.s0, p.wl_, p.sl_
    grads = p.grads
    del p
    torch.cuda.empty_cache()
    stream = torch.cuda.current_stream()
    dt = 0 if wl.dtype == "f32" else 1
    shape = (wl.n, wl.c, wl.h, wl.w)

    def peak(fn):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    def fused_step():
        wt.wtconv_forward(x, w0, b0, s0, wl_, sl_, y=y, stream=stream)
        wt.wtconv_backward_data(dy, w0, s0, wl_, sl_, dx=dx, stream=stream)
        n = wt.wtconv_workspace_size(shape, wl.k, wl.levels, dt, _native.OP_BWD_WEIGHT)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
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
        for op in ops:
            op()
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
    del ws
    torch.cuda.empty_cache()
    return {"us_ops": med, "steps": steps, "peak_mem_fused_bytes": int(mem_fused),
            "peak_mem_unfused_bytes": int(mem_unfused)}


def counter_op(args, wl):
    """Only one op, reps + 1 times (the first one warm), on one workload: the
    program the counter runs profile."""
    import torch

    import level_haar_wavelet_amd as wt
    from level_haar_wavelet_amd import _native
    from level_haar_wavelet_amd import unfused as uf

    _native.load()
    p = make_points([wl])[0]
    stream = torch.cuda.current_stream()
    if args.counter_op == "unfused_fwd":
        ws = uf.workspace(p.x, wl.k, wl.levels)
        op = lambda: uf.wtconv_unfused_forward(p.x, p.w0, p.b0, p.s0, p.wl_, p.sl_, ws, y=p.y, stream=stream)
    else:
        op = p.ops(stream)[("fwd", "bwd_data", "bwd_weight").index(args.counter_op)]
    for _ in range(args.reps + 1):
        op()
    torch.cuda.synchronize()
    print(json.dumps({"counter_op": args.counter_op, "workload": workload_name(wl), "calls": args.reps + 1}))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _oracle_pass(oracle, inp, wl, threads):
    args = (inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels)
    oracle.forward(inp.x, *args, nthreads=threads)
    oracle.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels, nthreads=threads)
    oracle.backward_weight(inp.x, inp.dy, *args, nthreads=threads)


def cpu_baseline(wls, images, single_thread=(), min_seconds=0.0):
    """The CPU oracle (as it stands) on a bounded sample: `images` images of
    every workload point in `wls`, one forward, data backward and weight
    backward each (repeated until `min_seconds` have passed); the rate is the
    sample's own modeled bytes (6 E e per pass) over the time.  Also a
    one-thread time of one pass for each workload in `single_thread`."""
    import oracle
    from level_haar_wavelet_amd.synthetic import make_inputs

    threads = oracle.default_threads()
    try:
        threads = min(threads, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    samples = []
    for wl in wls:
        n = max(1, min(images, wl.n))
        samples.append((wl, n, make_inputs(n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)))
    wl0, _, inp0 = samples[0]
    one = make_inputs(1, 1, 8, 8, wl0.k, wl0.levels, seed=0)
    _oracle_pass(oracle, one, dataclasses.replace(wl0, n=1, c=1, h=8, w=8), 1)  # load outside the timing
    passes, nbytes, t0 = 0, 0.0, time.perf_counter()
    while True:
        for wl, n, inp in samples:
            _oracle_pass(oracle, inp, wl, threads)
            nbytes += 6.0 * n * wl.c * wl.h * wl.w * wl.ebytes
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 50:
            break
    names = sorted({"%s L=%s" % (wl.name, ",".join(str(w.levels) for w in wls if w.name == wl.name)) for wl in wls})
    out = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": "%d image(s) of each of %d point(s) (%s, %s), fwd + bwd_data + bwd_weight in fp64, %d pass(es), "
                     "%.2f s wall" % (samples[0][1], len(samples), "; ".join(names),
                                      "/".join(sorted({w.dtype for w in wls})), passes, dt),
           "seconds": round(dt, 3)}
    one_thread = {}
    for wl in single_thread:
        inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
        t1 = time.perf_counter()
        _oracle_pass(oracle, inp, wl, 1)
        dt1 = time.perf_counter() - t1
        one_thread[wl.name] = {"seconds_per_pass": round(dt1, 4),
                               "GBs": round(6.0 * wl.elems * wl.ebytes / dt1 / 1e9, 4)}
    if one_thread:
        out["one_thread"] = one_thread
    return out


def graph_step_ms(torch, step, warmup, steps):
    """The same step captured once in a HIP graph and replayed: K replays timed
    between two events, after W untimed ones.  Returns ms per step, or the
    error text if capture fails."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
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


def selected_workloads(args):
    from level_haar_wavelet_amd.synthetic import WORKLOADS, sweep_workloads

    if args.workload == "sweep" and args.levels is None and args.dtype is None:
        return sweep_workloads()
    wl = WORKLOADS[args.workload]
    if args.levels is not None or args.dtype is not None:
        wl = wl.with_levels(args.levels if args.levels is not None else wl.levels, args.dtype)
    return [wl]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ramp-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="sweep")
    ap.add_argument("--levels", type=int, default=None)
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--cpu-sample", type=int, default=4, help="images per point of the CPU-oracle sample (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU-oracle sample until this much wall time has passed")
    ap.add_argument("--mall-flush", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--counter-op", default=None, choices=sorted(OP_KEYS))
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--trace-summary", default=None)
    ap.add_argument("--traffic-summary", default=None)
    ap.add_argument("--valu-summary", default=None)
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-baseline comparison")
    ap.add_argument("--no-comparator", action="store_true", help="skip the 7x7 depthwise comparator")
    ap.add_argument("--no-extra", action="store_true", help="skip the stage1 and large-workload lines")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (graph_ms_per_step)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU layer; more than one GPU is not supported in this build "
              "(every workload fits one GPU, and the layer needs no collective for its forward or data "
              "backward; the design notes describe how it would shard).", file=sys.stderr)
        sys.exit(2)

    wls = selected_workloads(args)
    if args.trace_summary:
        print(trace_summary(args.trace_summary, wls[0]))
        return
    if args.traffic_summary:
        print(json.dumps(traffic_summary(args.traffic_summary, wls[0], args.reps, args.copy_calibration or (1 << 30)),
                         indent=1))
        return
    if args.valu_summary:
        print(valu_summary(args.valu_summary, wls[0], args.reps))
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
    if args.counter_op:
        counter_op(args, wls[0])
        return

    import torch

    from level_haar_wavelet_amd import _native
    from level_haar_wavelet_amd.synthetic import WORKLOADS

    _native.load()
    torch.cuda.set_device(0)
    points = make_points(wls)
    ms, res = time_points(args, points)
    graph = None
    if args.graph and not args.mall_flush:
        stream = torch.cuda.current_stream()
        allops = [op for p in points for op in p.ops(stream)]
        graph = graph_step_ms(torch, lambda: [op() for op in allops], args.warmup, args.steps)
    del points
    torch.cuda.empty_cache()
    step_bytes = sum(6.0 * wl.elems * wl.ebytes for wl in wls)
    value = step_bytes / (ms * 1e-3) / 1e9
    digest = source_digest()
    # the dominant op: the longest mean duration of any op at any point
    dom = max(((i, j) for i in range(len(wls)) for j in range(3)), key=lambda ij: res[ij[0]]["us_ops_mean"][ij[1]])
    rl = roofline(wls[dom[0]], OPS[dom[1]], res[dom[0]]["us_ops_mean"][dom[1]], digest)
    wl0 = wls[0]
    sweep = len(wls) > 1
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": ("level sweep 32x128x128x128 k=5, L=1..5, fp32 and fp16 storage (ten points, "
                                "one step = fwd + bwd_data + bwd_weight at every point)") if sweep
                   else workload_name(wl0),
                   "n": wl0.n, "c": wl0.c, "h": wl0.h, "w": wl0.w, "k": wl0.k,
                   "levels": sorted({w.levels for w in wls}), "storage": sorted({w.dtype for w in wls}),
                   "arithmetic": "fp32", "parallelism": "single GPU"},
        "value_is": "sum over the points of the modeled minimum bytes 6 E e (fwd 2 E e, bwd_data 2 E e, "
                    "bwd_weight 2 E e) / the step time",
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "points": [point_record(w, r) for w, r in zip(wls, res)],
        "us_per_op": "medians over the timed steps of HIP events around each call",
        "stream_copy_GBs": round(stream_copy_gbs(), 1),
        "modeled_bytes_per_step": step_bytes,
        "mall_flush": bool(args.mall_flush),
        "roofline": rl,
    }
    if graph is not None:
        line["graph_ms_per_step"] = round(graph["ms_per_step"], 4) if "ms_per_step" in graph else graph.get("error")
    if not args.no_extra and sweep:
        # the other workloads, one step each, timed the same way
        extra = {}
        for name in ("stage1", "stage2", "large"):
            wl = WORKLOADS[name]
            ms2, r2 = time_points(args, make_points([wl]))
            torch.cuda.empty_cache()
            rec = point_record(wl, r2[0])
            rec["workload"] = workload_name(wl)
            rec["roofline_frac_dominant"] = roofline(wl, OPS[max(range(3), key=lambda j: r2[0]["us_ops_mean"][j])],
                                                     max(r2[0]["us_ops_mean"]), digest)["frac"]
            extra[name] = rec
        line["other_workloads"] = extra
    if not args.no_extra and sweep:
        # dx and every gradient in one call: fused where a plane fits one
        # workgroup (stage1, stage2), the two calls elsewhere (the sweep)
        fb = {}
        for name in ("stage1", "stage2"):
            rec = extra[name]
            us = time_backward(args, WORKLOADS[name])
            torch.cuda.empty_cache()
            two = rec["us_bwd_data"] + rec["us_bwd_weight"]
            fb[name] = {"us_backward": round(us, 2), "us_bwd_data_plus_bwd_weight": round(two, 2),
                        "speedup": round(two / us, 3),
                        "GBs_modeled_5Ee": round(5.0 * WORKLOADS[name].elems * WORKLOADS[name].ebytes / (us * 1e-6)
                                                 / 1e9, 1)}
        line["fused_backward"] = {"what": "the single fused backward pass (wtconv_backward with WTCONV_FUSED_BWD=1: "
                                          "x and dy read once, dx and all gradients written) against "
                                          "wtconv_backward_data + wtconv_backward_weight (the default)", **fb}
    if not args.no_unfused and sweep:
        line["block_peak_memory"] = {name: block_memory(WORKLOADS[name]) for name in ("stage1", "stage2")}
        torch.cuda.empty_cache()
    ref = wls[min(2, len(wls) - 1)] if sweep else wl0  # the L = 3 fp32 point of the sweep
    if not args.no_unfused:
        u = run_unfused(args, ref)
        r = next(rr for w, rr in zip(wls, res) if w == ref)
        uf, ub, uw = u["us_ops"]
        us_f, us_b, us_w = r["us_ops"]
        line["unfused_baseline"] = {
            "what": "the same layer as separate kernels with every intermediate in HBM (wtconv_unfused_*), "
                    "timed the same way (medians over %d steps)" % u["steps"],
            "workload": workload_name(ref),
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
        cmp_ = {}
        for w in ([ref, next((w for w in wls if w.dtype == "f16" and w.levels == ref.levels), None)]
                  if sweep else [ref]):
            if w is None:
                continue
            dw = dataclasses.replace(w, name=w.name, k=7, levels=0)
            _, r7 = time_points(args, make_points([dw]))
            torch.cuda.empty_cache()
            f7, b7, w7 = r7[0]["us_ops"]
            r = next(rr for ww, rr in zip(wls, res) if ww == w)
            us_f, us_b, us_w = r["us_ops"]
            cmp_[w.dtype] = {"workload": workload_name(w), "us_fwd": round(f7, 2), "us_bwd_data": round(b7, 2),
                             "us_bwd_weight": round(w7, 2), "us_fwd_bwd": round(f7 + b7 + w7, 2),
                             "wtconv_over_dw7x7_fwd": round(us_f / f7, 3),
                             "wtconv_over_dw7x7_fwd_bwd": round((us_f + us_b + us_w) / (f7 + b7 + w7), 3)}
        line["dw7x7_comparator"] = {"what": "7x7 depthwise conv (+bias, scale) on the same tensors, same timing; "
                                            "98 FLOP per element against WTConv's 2 k^2 (1 + S(L))", **cmp_}
    if args.cpu_sample > 0:
        single = [WORKLOADS[n] for n in ("tiny", "stage1", "stage2")] if sweep else []
        line["cpu_baseline"] = cpu_baseline(wls, args.cpu_sample, single_thread=single, min_seconds=args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
