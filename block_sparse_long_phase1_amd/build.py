"""Compile libstarattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libstarattn.so")
# Profiling build: the same library with decode.hip compiled with STAR_DECODE_TIMELINE
# (per-workgroup timestamps of each decode launch; read by decode_timeline.py).
TIMELINE_LIB_PATH = os.path.join(PKG, "libstarattn_timeline.so")
TIMELINE_SOURCE = "decode.hip"
ARCH = os.environ.get("STAR_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU ops stay disabled: the kernels' fp32 math is written as scalar code.  Host
# symbols are hidden except the C entry points (STAR_API in the header).
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fvisibility=hidden",
               "-I" + INCLUDE, "-I" + CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _link(hipcc: str, objs: list[str], out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object under _build/ and link libstarattn.so, and the
    profiling library libstarattn_timeline.so.  Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    timeline_src = os.path.join(CSRC, TIMELINE_SOURCE)
    units = [(src, os.path.basename(src) + ".o", []) for src in srcs]
    units.append((timeline_src, TIMELINE_SOURCE + ".timeline.o", ["-DSTAR_DECODE_TIMELINE"]))

    def compile_one(unit) -> str:
        src, name, extra = unit
        obj = os.path.join(BUILD_DIR, name)
        cmd = [hipcc, "-x", "hip", "-c", src, "-o", obj] + HIPCC_FLAGS + extra
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, res.stderr))
        if verbose:
            print(" ".join(cmd))
        return obj

    jobs = jobs or min(len(units), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, units))
    _link(hipcc, objs[:len(srcs)], LIB_PATH)
    _link(hipcc, [o for o, (src, _, _) in zip(objs[:len(srcs)], units) if src != timeline_src] + [objs[-1]],
          TIMELINE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
