"""The oracle's pins, re-run against a build of oracle.c with AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

The pins exercise every oracle entry point, including the skipped-entry and
skipped-slot paths, so an out-of-bounds read or write, a use of freed memory
or undefined arithmetic anywhere on those paths stops the run with a report.
The sanitised library is built beside the plain one (liboracle_san.so) and
loaded into a child interpreter that preloads the sanitizer runtimes.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_format.py", "tests/test_oracle_decode.py", "tests/test_oracle_fp8.py",
        "tests/test_oracle_staged.py", "tests/test_oracle_mtp.py", "tests/test_oracle_topk.py"]


def _runtime(name: str) -> str:
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""


def test_oracle_pins_under_address_and_ub_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    env = dict(os.environ)
    env.update(SMLA_ORACLE_SANITIZE="1", LD_PRELOAD=asan + ":" + ubsan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    build = subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stdout + build.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    for marker in ("AddressSanitizer", "runtime error:", "LeakSanitizer"):
        assert marker not in r.stdout + r.stderr, report
