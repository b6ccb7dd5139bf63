"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the native block pool (paged_kv_cache_72_amd/csrc/pa_blocks.cpp) and
the C oracle (oracle/oracle.c) are compiled with gcc/g++ and both sanitizers,
linked into the stress drivers under tests/sanitize/, and run; the drivers
call every entry point through seeded random operation sequences.  Any
invalid access, leak or undefined behaviour aborts the driver.  No GPU code
is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _build_and_run(cmd, exe):
    os.makedirs(OUT, exist_ok=True)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_pool_under_asan_ubsan():
    src = [os.path.join(ROOT, "tests", "sanitize", "bp_stress.cpp"),
           os.path.join(ROOT, "paged_kv_cache_72_amd", "csrc", "pa_blocks.cpp")]
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), *src]
    assert "bp_stress ok" in _build_and_run(cmd, os.path.join(OUT, "bp_stress"))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan():
    src = [os.path.join(ROOT, "tests", "sanitize", "oracle_stress.c"),
           os.path.join(ROOT, "oracle", "oracle.c")]
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-I",
           os.path.join(ROOT, "oracle"), *src, "-lm"]
    assert "oracle_stress ok" in _build_and_run(cmd, os.path.join(OUT, "oracle_stress"))
