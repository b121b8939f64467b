"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

``oracle.c`` is compiled by gcc with ``-fsanitize=address,undefined`` (every
undefined-behaviour report fatal) into a library of its own, and the
small-case oracle pins run against it in a child interpreter that preloads
the address-sanitizer runtime (leak checks off: the interpreter keeps its
own allocations to the end by design).  An out-of-bounds access, a use after
free, a signed overflow, a bad shift or a misaligned access anywhere in the
oracle's layout, dispatch, cached dispatch, combine, FP8 quantiser,
low-latency and relay code paths fails the run.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
FILES = ["tests/test_oracle_layout_dispatch.py", "tests/test_oracle_ll.py", "tests/test_oracle_relay.py",
         "tests/test_oracle_next.py", "tests/test_oracle_fuzz.py", "tests/test_golden.py"]
SUBSET = "not full_size and not large and not accuracy"   # the small cases: every oracle function, seconds each


def _runtime(name):
    if shutil.which("gcc") is None:
        return None
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's address-sanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-ffp-contract=off", "-shared", "-fPIC", "-o", lib, SRC, "-lm"])
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-k", SUBSET] + FILES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out
