"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/c/oracle_sanitize.c`` replays the hand-worked fixtures of
``tests/golden/`` through ``oracle/oracle.c`` and runs every oracle entry point
on ragged shapes with exact-size heap buffers, one and several threads,
degenerate sizes and rejected arguments.  Both are built here with gcc and the
sanitizers (host code only: no GPU and no HIP compiler involved); any
out-of-bounds access, leak or undefined operation aborts the program.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [gcc, "-O1", "-g", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math", *SAN,
           "-pthread", os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(HERE, "c", "oracle_sanitize.c"), "-o", exe, "-lm"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0 and ("asan" in p.stderr.lower() or "ubsan" in p.stderr.lower()):
        pytest.skip("sanitizer runtime not available: " + p.stderr[-300:])
    assert p.returncode == 0, p.stderr
    return exe


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe, os.path.join(HERE, "golden")], capture_output=True, text=True,
                       env=env, timeout=300)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-4000:]
    assert "0 failures" in p.stdout
    n = int(p.stdout.split()[0])
    assert n > 100000, p.stdout  # the golden cases and the full bf16 sweep ran
