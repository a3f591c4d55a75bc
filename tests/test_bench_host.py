"""Host-side logic of bench.py (no GPU): the single-GPU contract, the FLOP and
byte models the roofline is computed from, the counter-summary digest gate and
the CPU-oracle baseline leg."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from level_haar_wavelet_amd.synthetic import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "single-GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("levels,flop", [(1, 100.0), (2, 112.5), (3, 115.625), (4, 116.40625), (5, 116.6015625)])
def test_flops_per_element_follow_the_level_sum(levels, flop):
    """2 k^2 (1 + S(L)) FLOP per element with S(L) = sum 4^(1-l): k = 5 gives
    100, 112.5, 115.6, 116.4, 116.6 for L = 1..5 (one k x k MAC per base pixel,
    four bands of a quarter as many pixels per level)."""
    wl = WORKLOADS["sweep"].with_levels(levels, "f32")
    assert bench.conv_flops(wl) == pytest.approx(flop * wl.elems, rel=1e-12)


def test_modeled_step_bytes_are_six_tensor_moves():
    """Forward and data backward read one tensor and write one; the weight
    backward reads two: 6 E e per step (462 MB at stage1 in fp32)."""
    wl = WORKLOADS["stage1"]
    assert 6 * wl.elems * wl.ebytes == 64 * 96 * 56 * 56 * 4 * 6 == 462422016


def test_counter_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = bench.source_digest()
    wname = bench.workload_name(WORKLOADS["stage1"])
    (prof / "hbm_traffic.json").write_text(json.dumps(
        {wname: {"source_digest": digest, "ops": {"wtconv_forward": {"bytes_per_launch": 123.0}}}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wtconv_forward", digest, wname) == 123.0
    assert bench.measured_traffic("wtconv_forward", "0" * 16, wname) is None
    assert bench.measured_traffic("wtconv_backward_weight", digest, wname) is None
    # counters of another workload are not this one's
    assert bench.measured_traffic("wtconv_forward", digest, bench.workload_name(WORKLOADS["stage2"])) is None


def test_cpu_baseline_times_the_oracle_on_a_bounded_sample():
    wl = WORKLOADS["tiny"]
    out = bench.cpu_baseline([wl, wl.with_levels(1)], images=1, single_thread=[wl])
    assert out["kind"] == "oracle" and out["cores"] >= 1 and out["value"] > 0
    assert out["sample"].startswith("1 image(s) of each of 2 point(s)")
    assert out["cpu_model"] and out["one_thread"]["tiny"]["seconds_per_pass"] > 0


@pytest.mark.parametrize("name,levels,dtype,bound", [("stage1", 3, "f32", "hbm"), ("sweep", 5, "f32", "hbm"),
                                                     ("sweep", 1, "f16", "alu"), ("large", 4, "f16", "alu")])
def test_roofline_bound_follows_the_intensity_against_the_published_ridge(name, levels, dtype, bound):
    """fp32 storage: 100-117 FLOP per 8 bytes (12.5-14.6 FLOP/B) is below the
    ridge of 157.3 TFLOP/s over 8 TB/s (19.7 FLOP/B), so HBM bounds it; fp16
    storage halves the bytes (25-29 FLOP/B) and the fp32 vector ALUs bound it."""
    wl = WORKLOADS[name].with_levels(levels, dtype)
    r = bench.roofline(wl, "wtconv_forward", 100.0, "0" * 16)
    assert r["bound"] == bound
    if bound == "hbm":
        assert r["unit"] == "GB/s" and r["peak"] == 8000.0
        assert r["achieved"] == pytest.approx(2 * wl.elems * wl.ebytes / 1e-4 / 1e9, rel=1e-3)
    else:
        assert r["unit"] == "TFLOP/s" and r["peak"] == 157.3
        assert r["achieved"] == pytest.approx(bench.conv_flops(wl) / 1e-4 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["nonpacked_fp32_frac"] == pytest.approx(r["achieved_TFLOPs"] / 78.6432, rel=1e-3)


def test_unfused_byte_model_matches_the_pages_endpoints():
    """The unfused forward moves (7 + 10.75 S(L)) E elements: 17.75 E at L = 1
    and 21.32 E at L = 5, the two ends the pages give for the reference."""
    wl1 = WORKLOADS["sweep"].with_levels(1, "f32")
    wl5 = WORKLOADS["sweep"].with_levels(5, "f32")
    assert bench.unfused_forward_elements(wl1) / wl1.elems == pytest.approx(17.75)
    assert bench.unfused_forward_elements(wl5) / wl5.elems == pytest.approx(21.32, abs=0.01)


def test_source_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "k.hip").write_text("int f(int a) { return a * 2; }  // doubles\n")
    (src / "k.h").write_text("/* header */\n#define N 4\n")
    monkeypatch.setattr(bench, "CSRC", str(src))
    d0 = bench.source_digest()
    (src / "k.hip").write_text("// a new comment\nint f(int a)\n{\n    return a * 2;  /* doubles */\n}\n")
    assert bench.source_digest() == d0
    (src / "k.hip").write_text("int f(int a) { return a * 3; }\n")
    assert bench.source_digest() != d0


def _write_counters(folder, rows):
    import csv

    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)  # quotes the kernel names, which hold commas
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_traffic_summary_sums_an_ops_launches_and_scales_by_the_copy(tmp_path):
    # a 1 MiB copy whose FETCH_SIZE reads half its bytes (factor 2) and whose
    # WRITE_SIZE reads them exactly (factor 1); the op runs twice (reps = 1),
    # two kernels per call
    copy = 1 << 20
    whole, low = "wtconv_whole_kernel<float, 5, 4, true, false>", "lowpass_kernel<float>"
    _write_counters(tmp_path / "fwd_fetch", [(1, "void %s(WtcWholeArgs<float>)" % low, "FETCH_SIZE", 100),
                                             (2, whole, "FETCH_SIZE", 300), (3, low, "FETCH_SIZE", 100),
                                             (4, whole, "FETCH_SIZE", 300), (5, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 7)])
    _write_counters(tmp_path / "fwd_write", [(1, low, "WRITE_SIZE", 10), (2, whole, "WRITE_SIZE", 30),
                                             (3, low, "WRITE_SIZE", 10), (4, whole, "WRITE_SIZE", 30)])
    _write_counters(tmp_path / "cfetch", [(1, "copyBuffer", "FETCH_SIZE", 512)])
    _write_counters(tmp_path / "cwrite", [(1, "copyBuffer", "WRITE_SIZE", 1024)])
    wl = WORKLOADS["stage1"]
    out = bench.traffic_summary(str(tmp_path), wl, 1, copy, outdir=str(tmp_path))
    assert out["fetch_factor"] == pytest.approx(2.0) and out["write_factor"] == pytest.approx(1.0)
    op = out["ops"]["wtconv_forward"]
    assert op["fetch_bytes"] == pytest.approx(400 * 1024 * 2.0)
    assert op["write_bytes"] == pytest.approx(40 * 1024)
    assert op["bytes_per_launch"] == pytest.approx((800 + 40) * 1024)
    assert op["kernels"][low]["dispatches"] == pytest.approx(1.0)
    assert "__amd_rocclr_copyBuffer" not in op["kernels"]
    assert out["source_digest"] == bench.source_digest()
    saved = json.load(open(tmp_path / "hbm_traffic.json"))
    assert saved == {out["workload"]: json.loads(json.dumps(out))}
    out2 = bench.traffic_summary(str(tmp_path), WORKLOADS["stage2"], 1, copy, outdir=str(tmp_path))
    saved = json.load(open(tmp_path / "hbm_traffic.json"))
    assert set(saved) == {out["workload"], out2["workload"]}
    assert (tmp_path / "stage1_hbm_traffic.md").read_text().count("rocprofv3 --pmc") == 4


@pytest.mark.parametrize("raw, short", [
    ("_Z19wtconv_whole_kernelIDF16_Li5ELi4ELb1EEv12WtcWholeArgsIT_E", "wtconv_whole_kernel<_Float16, 5, 4, true>"),
    ("_Z19wtconv_wgrad_kernelIfLi5ELi4ELi3ELb0EEv12WtcWgradArgsIT_E", "wtconv_wgrad_kernel<float, 5, 4, 3, false>"),
    ("_ZN12_GLOBAL__N_114lowpass_kernelIDF16_EEvPKT_PS1_lii", "lowpass_kernel<_Float16>"),
    ("void wtconv_whole_kernel<float, 5, 4, false>(WtcWholeArgs<float>)", "wtconv_whole_kernel<float, 5, 4, false>"),
    ("wtconv_wgrad_finalize_kernel(int, int, float const*)", "wtconv_wgrad_finalize_kernel"),
    ("__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"),
    ("void (anonymous namespace)::lowpass_kernel<float>(float const*, float*, long, int, int)",
     "lowpass_kernel<float>"),
])
def test_profiler_kernel_names_are_shortened(raw, short):
    assert bench._short_kernel(raw) == short
