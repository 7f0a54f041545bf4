"""The host launch plan over extreme requests (no GPU needed).

tests/plan_host.hip compiles the library's host source with stubbed kernel
entry points and drives its planning function over k up to 2^31 - 1, one to
2^31 - 1 segments, every ordering and several segment-size hints: every plan
must come back (no endless loop in the size arithmetic), with dynamic LDS,
stash, grid and scratch sizes inside their limits.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not found")
def test_plans_for_extreme_requests(tmp_path):
    exe = tmp_path / "plan_host"
    subprocess.check_call([HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(HERE, "plan_host.hip"), "-o", str(exe)],
                          stderr=subprocess.DEVNULL)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "bad: 0" in r.stdout
