"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

kvc_oracle.c is rebuilt with gcc's address and undefined-behaviour checks
(any report aborts), and every pin file runs against that build in a
subprocess: an out-of-bounds read or write, a signed overflow or a bad shift
anywhere the pins reach fails the test.  The sanitizer runtime is preloaded
because the library is loaded into an uninstrumented Python through ctypes.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvc_oracle.c")
PINS = ["test_oracle_pins.py", "test_oracle_swa_pins.py", "test_oracle_store_pins.py", "test_oracle_online_pins.py",
        "test_oracle_page4_pins.py"]


def _runtime(name):
    path = subprocess.check_output(["gcc", "-print-file-name=" + name]).decode().strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = tmp_path / "libkvc_oracle_sanitized.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(lib), SRC, "-lm"])
    env = dict(os.environ, KVC_ORACLE_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"]
                       + [os.path.join(ROOT, "tests", f) for f in PINS],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=900)
    out = r.stdout.decode(errors="replace")
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
