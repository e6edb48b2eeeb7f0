"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with the host compilers (g++ / gcc, never hipcc) and run:

* tests/sanitize/host_plan_check.cpp with block_sparse_long_phase1_amd/csrc/host_plan.cpp: the
  library's host-side planning (decode chunk plan, Phase-2 split plan, workspace carve-up) and
  its argument checks, over thousands of seeded random shapes and the edges (64 shards, empty
  shards, tail_len = 0, contexts at the 2^24-token limit);
* tests/sanitize/oracle_check.c with oracle/star_oracle.c: the fp64 oracle over seeded random
  small shapes, every input type, sampled rows, causal and empty partitions, merges.

Each program checks its own invariants; a sanitizer report or a failed check makes it exit
non-zero.  The two builds share no source.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_phase1_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _compiler(name):
    cc = shutil.which(name)
    if cc is None:
        pytest.skip("%s not available" % name)
    return cc


def _run(cmd, exe, tmp_path):
    build = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    assert build.returncode == 0, "build failed:\n%s" % build.stderr[-4000:]
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=240)
    assert res.returncode == 0, "sanitized run failed (%d):\n%s\n%s" % (res.returncode, res.stdout[-2000:],
                                                                        res.stderr[-6000:])
    assert res.stdout.strip().splitlines()[-1].startswith("ok:"), res.stdout
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
    return res.stdout


def test_host_plan_and_argument_checks_sanitized(tmp_path):
    cxx = _compiler("g++")
    exe = str(tmp_path / "host_plan_check")
    cmd = [cxx, "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                                       "-I/opt/rocm/include", "-I" + CSRC, os.path.join(CSRC, "host_plan.cpp"),
                                       os.path.join(ROOT, "tests", "sanitize", "host_plan_check.cpp"), "-o", exe]
    out = _run(cmd, exe, tmp_path)
    assert "3000 decode plans" in out


def test_oracle_sanitized(tmp_path):
    cc = _compiler("gcc")
    exe = str(tmp_path / "oracle_check")
    cmd = [cc, "-std=c99"] + SAN + ["-pthread", os.path.join(ROOT, "oracle", "star_oracle.c"),
                                    os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-o", exe, "-lm"]
    out = _run(cmd, exe, tmp_path)
    assert "phase-1 calls" in out
