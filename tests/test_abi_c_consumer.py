"""The boundary is a C ABI: a plain C99 program (tests/c_abi_consumer.c) includes
include/star_attn.h, links libstarattn.so and calls its host-side entry points (status
strings, workspace queries, argument checks that fail before any HIP call).  CPU only."""
import os
import shutil
import subprocess

import pytest

import block_sparse_long_phase1_amd as sa
from block_sparse_long_phase1_amd import build as sa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_uses_the_abi(tmp_path):
    if not os.path.exists(sa.LIB_PATH):
        sa_build.build()
    libdir = os.path.dirname(sa.LIB_PATH)
    exe = str(tmp_path / "c_abi_consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_consumer.c"), "-o", exe,
           "-L" + libdir, "-lstarattn", "-Wl,-rpath," + libdir, "-L" + os.path.join(ROCM, "lib"),
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, capture_output=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    lines = run.stdout.strip().splitlines()
    assert run.returncode == 0, run.stdout + run.stderr
    assert len(lines) >= 16 and all(line.startswith("ok") for line in lines), run.stdout
