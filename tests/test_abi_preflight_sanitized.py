"""The C ABI's host-side preflight under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; the kernels are built as usual).

preflight_fuzz.cpp calls every entry point with fuzzed sizes, strides, group
sizes, leading dimensions and eps values, and fake pointers: null, misaligned,
overlapping, far apart, at the top of the address space.  Every call must
return a status, with no sanitizer report, and every status the preflight can
give must occur.  The preflight only compares pointer values, never reads
through them; with no GPU visible a call that passes it stops at the device
check before any launch, and the driver refuses to run where a GPU is visible.
"""

import os
import re
import subprocess

import pytest

from rmsnorm_activation_quantization_amd import _build

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def test_preflight_fuzz_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "preflight_fuzz")
    cmd = [_build.HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SANITIZE,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(_build.SOURCE),
           os.path.join(TESTS, "preflight_fuzz.cpp"), _build.SOURCE, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"}
    run = subprocess.run([exe, "300000"], capture_output=True, text=True, timeout=600, env=env)
    if run.returncode == 2 and "GPU is visible" in run.stderr:
        pytest.skip("a GPU is visible: the fuzz passes fake pointers and runs only without one")
    out = run.stdout + run.stderr
    assert run.returncode == 0 and "runtime error" not in out and "Sanitizer" not in out, out[-4000:]
    counts = dict(re.findall(r"(ok|invalid|unsupported|hip|device) (\d+)", out))
    assert set(counts) == {"ok", "invalid", "unsupported", "hip", "device"}, out
    # empty batches, refusals of both kinds, and calls that pass the whole
    # preflight (stopped at the device check: no GPU here)
    assert all(int(counts[k]) > 0 for k in ("ok", "invalid", "unsupported", "hip")), counts
