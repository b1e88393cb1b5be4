"""The oracle's pins run against an AddressSanitizer + UndefinedBehaviorSanitizer
build of the oracle (host code only), in a child process with the sanitizer
runtimes preloaded: an out-of-bounds access, a use after free or undefined
arithmetic anywhere in the C the pins exercise fails this test."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_pins.py", "test_oracle_bwd_pins.py", "test_oracle_conv_pins.py",
        "test_oracle_ssd_pins.py", "test_oracle_disc_pins.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    so = oracle.build_sanitized()
    # the sanitizer runtimes must come first; anything already preloaded stays
    pre = ":".join(p for p in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if p)
    env = dict(os.environ, SSM_ORACLE_LIB=so, LD_PRELOAD=pre,
               # the interpreter's own allocations are not the oracle's to answer for
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report goes to stderr as the child aborts; keep it visible
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", f) for f in PINS]]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
