"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run through the quick pins in a child process
(the same inputs that catch the planted mutants: worked streams, round trips
on the workloads, edge values, corrupt and truncated streams, split records,
interleaved containers, the table builder and the front end).  Any
out-of-bounds access, use of freed memory, signed overflow, bad shift or
other undefined operation aborts the child and fails the test.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RUNNER = os.path.join(HERE, "mutant_runner.py")
SANITIZE = ("-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_sanitized_oracle_passes_the_pins(tmp_path):
    libasan = _runtime("libasan.so")
    if libasan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = str(tmp_path / "librans_oracle_sanitized.so")
    oracle.build(out=lib, extra_flags=SANITIZE)
    # the interpreter is not instrumented, so the ASan runtime is preloaded;
    # leak checking is off (the interpreter's own allocations would show)
    env = dict(os.environ, LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, RUNNER, lib], env=env, capture_output=True, text=True,
                         timeout=900)
    assert res.returncode == 0, (res.stdout[-3000:] + "\n" + res.stderr[-6000:])
