"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two drivers in tests/sanitize/ are built with the sanitizers on their host
code and run:
  * oracle_driver.c with oracle.c (gcc): every oracle entry on small random
    inputs with out-of-range lengths, masks, invalid and duplicate list
    entries, step rows, INT8 pages with ids outside the pool, appends past
    the capacity and top-k over ties, NaN and infinities;
  * host_driver.cpp with the HIP library sources (hipcc; the sanitizers
    apply to the host code only, -Xarch_host before each option): launch
    planning over a grid of shapes with its documented invariants, the
    gather-or-scan choice, top-k planning and argument validation of every
    entry point (no GPU needed: valid calls stop at the device query).
Any out-of-bounds access, use after free or undefined arithmetic aborts the
run, and the drivers' own checks must pass."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-pthread", os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True, capture_output=True)
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_driver")
    csrc = os.path.join(ROOT, "decode_attention_flash_amd", "csrc")
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           os.path.join(csrc, "ck_decode_attn.hip"), os.path.join(csrc, "ck_topk.hip"),
           os.path.join(HERE, "host_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=900, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
