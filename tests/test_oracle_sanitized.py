"""The oracle's C built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host
code only), and every oracle pin run against that build in a child process: an
out-of-bounds access, a use of freed memory or undefined behaviour (signed overflow, bad
shift, misaligned access) anywhere on the paths the pins reach fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "vq_oracle.c")


def _gcc_lib(name):
    try:
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        return None
    p = p.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _gcc_lib("libasan.so")
    if shutil.which("gcc") is None or asan is None:
        pytest.skip("gcc with AddressSanitizer is not available")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib, SRC, "-lm"], check=True, cwd=ROOT)
    env = dict(os.environ)
    env.update({"VQ_ORACLE_LIB": lib, "LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
