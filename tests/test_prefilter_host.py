"""The kernels' key transform and raw-bit bound test, checked on the host (no
GPU needed).

tests/prefilter_exact.hip includes the kernel header, builds host-only with
hipcc and checks, for every key type:
  * the order-preserving transform against numeric comparison of the keys as
    the compiler decodes them: a < b exactly when ord(a) < ord(b), a == b
    exactly when ord(a) == ord(b) (so -0.0 and +0.0 meet), over every 16-bit
    pattern and over boundary and a million seeded random 32-bit patterns;
  * for every direction, that the test built for each pass-0 bucket bound
    passes exactly the keys whose order-preserving bits are within the bound,
    and that the per-lane chunk reduction agrees with the per-key test.
Run with --perturbed, the same binary swaps in a transform with a planted
mistake and must catch it for every key type.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not found")
def test_raw_bit_bound_test_is_exact(tmp_path):
    exe = tmp_path / "prefilter_exact"
    subprocess.check_call([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(HERE, "prefilter_exact.hip"), "-o", str(exe)],
                          stderr=subprocess.DEVNULL)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "total mismatches: 0" in r.stdout
    assert r.stdout.count("ordered bits vs numeric order") == 7
    p = subprocess.run([str(exe), "--perturbed"], capture_output=True, text=True, timeout=300)
    print(p.stdout)
    assert p.returncode == 0 and "caught for 7 of 7" in p.stdout, p.stdout
