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
    (prof / "hbm_traffic.json").write_text(json.dumps(
        {"source_digest": digest, "kernels": {"wtconv_forward": {"bytes_per_launch": 123.0}}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wtconv_forward", digest) == 123.0
    assert bench.measured_traffic("wtconv_forward", "0" * 16) is None
    assert bench.measured_traffic("wtconv_backward_weight", digest) is None


def test_cpu_baseline_times_the_oracle_on_a_bounded_sample():
    wl = WORKLOADS["tiny"]
    out = bench.cpu_baseline(wl, images=1, min_seconds=0.05)
    assert out["kind"] == "oracle" and out["cores"] >= 1 and out["value"] > 0
    assert "1 of %d images" % wl.n in out["sample"]


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
