"""Builds the HIP library libsegtopk.so for gfx950 with hipcc (in-tree).

Every source under csrc/ (the host code and one kernel unit per key type) is
compiled to an object in parallel, then the objects are linked into one
shared library.  Objects go to a build folder beside the sources.  The
benchmark's stream-read probe (probe/stream_read.hip) is built alongside as
libsegtopk_probe.so; the top-k library does not use it.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsegtopk.so")
PROBE_SRC = os.path.join(HERE, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(HERE, "probe", "libsegtopk_probe.so")
ARCH = os.environ.get("SEGTOPK_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed-fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[hipcc, *HIPCC_FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    # The benchmark's stream-read probe: a library of its own.
    cmds.append([hipcc, *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", PROBE_LIB])
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds):
            if r.stderr and verbose:
                # hipcc's host pass warns about the device-only feature flag.
                lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
                if lines:
                    print("\n".join(lines), flush=True)
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, r.args, r.stdout, r.stderr)
    tmp = LIB + ".tmp"
    link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
