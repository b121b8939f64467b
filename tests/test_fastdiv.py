"""The small kernels replace integer divides by a host-computed multiply-shift
(FastDiv in csrc/kernels.h, fdiv in csrc/device.h).  This builds a host-only
program from those headers and checks it against C integer division over every
range the kernels use: expert / experts-per-rank (both below 8192) and token /
tokens-per-channel for up to 2^20 tokens per source.  No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_get_dispatch_histogram_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_fastdiv_matches_integer_division(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    cmd = [HIPCC, "-O2", "-std=c++17", "-I" + CSRC, "-I" + os.path.join(ROOT, "include"),
           "--offload-arch=gfx950", "-x", "hip", os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok"), out.stdout
