"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): uzip_oracle.c is built with -fsanitize=address,undefined (UB
fatal), and the pins that drive its parsers hardest -- every named corruption,
the crafted over-long records, random byte flips of full- and sampled-table
frames, ragged round trips of every type, the arbitration frames -- run
against that build in a child process (UZIP_ORACLE_LIB; the sanitizer runtime
is preloaded there).  Any out-of-bounds access or undefined operation aborts
the child and fails this test."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "uzip_oracle.c")


def _runtime():
    try:
        p = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared", "-fPIC",
                               "-o", lib, SRC, "-lm"])
        env = dict(os.environ)
        env["UZIP_ORACLE_LIB"] = lib
        env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
               os.path.join(ROOT, "tests", "test_oracle_pins.py"),
               os.path.join(ROOT, "tests", "test_sampled_pins.py"),
               os.path.join(ROOT, "tests", "test_arbitration_pins.py"),
               "-k", "corruption or record or roundtrip or worked_example or empty or raw or realised or frames"]
        r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
        assert " passed" in r.stdout
