"""The host planners under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/planner_sweep.cpp against the library's sources with both
sanitizers on the host code (the gfx950 device code is built as usual and
never launched) and runs its
seeded sweep of valid and invalid descriptors (sides up to the longest
accepted, offsets past 2^32 elements, waves under small caps, overlaps).
Plan creation makes no HIP call, so this runs without a GPU.  To run it by
hand: ``python -m pytest tests/test_planner_sanitized.py -s``.
"""

import os
import subprocess

import pytest

from muon_newton_schulz_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_planner_sweep_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "planner_sweep")
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    cmd = [B.HIPCC, "--offload-arch=gfx950", "-x", "hip", "-O1", "-g", "-std=c++17",
           "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", B.CSRC,
           os.path.join(ROOT, "tests", "planner_sweep.cpp"), *srcs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-6000:])
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, \
        run.stderr[-6000:]
    ok, valid, rejected = run.stdout.split()
    assert ok == "ok" and int(valid) > 500 and int(rejected) > 250
