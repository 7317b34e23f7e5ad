"""Build the gfx950 attention library (``libattn09.so``) with hipcc.

Every ``csrc/*.hip`` file is compiled for gfx950 in parallel and linked into
one shared library next to this file; ``csrc/attn_sched_host.cpp`` (host code
over the work-decomposition functions, for the unit tests) goes into a small
library of its own.  Packed fp32 instructions are turned
off (``-packed-fp32-ops``); hipcc's host pass warns that it does not know the
feature, which is harmless.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn09.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# host-only library over the work-decomposition functions, for the unit tests
SCHED_LIB_PATH = os.path.join(HERE, "libattn09_sched.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _quiet(out: str) -> str:
    keep = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    return "\n".join(keep)


def build(verbose: bool = False, extra_flags=()) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, *extra_flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = _quiet(r.stdout + r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{_quiet(r.stdout + r.stderr)}")
    os.replace(tmp, LIB_PATH)
    build_sched(cc)
    return LIB_PATH


def build_sched(cc=None) -> str:
    """Compile attn_sched_host.cpp (host code only) into libattn09_sched.so."""
    cc = cc or hipcc()
    tmp = SCHED_LIB_PATH + ".tmp"
    cmd = [cc, "-x", "hip", "--cuda-host-only", f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-I", CSRC, os.path.join(CSRC, "attn_sched_host.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for attn_sched_host.cpp:\n{_quiet(r.stdout + r.stderr)}")
    os.replace(tmp, SCHED_LIB_PATH)
    return SCHED_LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
