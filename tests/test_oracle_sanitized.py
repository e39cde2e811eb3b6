"""The oracle's pins, run again against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of the oracle (host code only, gcc). Any out-of-bounds
access, use after free, signed overflow, invalid shift or out-of-range
float-to-int conversion in the oracle aborts the run."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_forward.py", "tests/test_oracle_blocks.py",
             "tests/test_oracle_drafter.py"]
SAN = ["-fsanitize=address,undefined", "-fsanitize=float-cast-overflow", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g"]


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    so = oracle.build(extra_flags=SAN, out=str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, SPECV_ORACLE_SO=so, LD_PRELOAD=f"{asan}:{ubsan}",
               # Python itself is not built with the sanitizers: its own
               # allocations would read as leaks at exit
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
