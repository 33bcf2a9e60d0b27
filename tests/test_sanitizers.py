"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI layer (capi.cpp: validation, overlap and alignment checks, error text, launch
planning) and the fp64 oracle (ssm_oracle.c) are rebuilt with -fsanitize=address,undefined
(selective_scan_02_amd.build.build_sanitized, oracle.build(sanitize=True)), and the ABI and
oracle test files are run again against those builds in a child process with gcc's ASan
runtime preloaded.  Any sanitizer report fails the child (UBSan is built non-recoverable,
ASan aborts on its first error), and the test also looks for report text.  No kernel is
launched: the ABI tests exercise the host paths, which return before any HIP call.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
def test_abi_and_oracle_tests_under_asan_ubsan():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan.so is not installed")
    import oracle
    from selective_scan_02_amd import build as b

    lib = b.build_sanitized(OUT)
    olib = oracle.build(force=True, out=os.path.join(OUT, "liboracle_asan.so"), sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        # the interpreter itself is not instrumented and never frees some of its memory
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "SSM_SCAN_LIB": lib,
        "SSM_ORACLE_LIB": olib,
        "HIP_VISIBLE_DEVICES": "",  # host paths only, also on a machine with a GPU
    })
    # the child maps the sanitized builds, with the ASan runtime active
    probe = ("import ctypes, oracle, selective_scan_02_amd as s; s.load(); oracle._load(); "
             "ctypes.CDLL(None).__asan_report_load1; maps = open('/proc/self/maps').read(); "
             "print('libssm_scan_asan.so' in maps, 'liboracle_asan.so' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.split() == ["True", "True"], r.stdout + r.stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert "passed" in r.stdout
