"""The oracle and the CPU emulation of the kernels built with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only) and run on small cases of
every kernel family against each other: any out-of-bounds access, leak-free
use-after-free, misaligned access or undefined arithmetic in the phase code or
the oracle aborts the run."""
import os
import subprocess

import pytest

from tests import emulation as emu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(not emu.available(), reason="no clang++ for the emulation")


def test_emulation_and_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    cxx = emu._compiler()
    cc = os.path.join(os.path.dirname(cxx), "clang")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    obj = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "sanitized")
    subprocess.run([cc, "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-c", os.path.join(ROOT, "oracle", "wtconv_oracle.c"),
                    "-o", obj] + san, check=True)
    subprocess.run([cxx, "-std=c++17", "-fno-strict-aliasing", "-o", exe,
                    os.path.join(ROOT, "tests", "emulation", "sanitize_main.cpp"), obj, "-pthread"] + san, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "all cases ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
