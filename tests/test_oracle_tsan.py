"""The oracle's protocol emulator under ThreadSanitizer (CPU only).

oracle/tsan_main.c drives orc_ag_gemm_protocol -- producer threads copying signal tiles and release-storing
their flags, consumer threads acquire-waiting on a panel's flags before reading it (Triton-distributed
semantics page, "Producer-consumer model", "Signal-based synchronization") -- over ranks, arrival orders,
seeds and delays.  Built with gcc -fsanitize=thread, the emulator must report no data race and reproduce the
plain oracle's C bit for bit; with its consumers' waits removed (a planted mistake) the sanitizer must report
the race.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.fixture(scope="module")
def tsan_bin(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("tsan") / "tsan_main")
    r = subprocess.run([gcc, "-fsanitize=thread", "-O1", "-g", "-std=c11", "-Wno-unknown-pragmas",
                        "-I" + ORACLE, os.path.join(ORACLE, "tsan_main.c"), "-o", out, "-lpthread", "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower():
        pytest.skip("ThreadSanitizer runtime not available: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    return out


def _run(binary, *args):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    return subprocess.run([binary, *args], capture_output=True, text=True, timeout=300, env=env)


def test_emulator_has_no_data_race(tsan_bin):
    r = _run(tsan_bin)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert "0 differ" in r.stdout


def test_planted_missing_wait_is_reported(tsan_bin):
    r = _run(tsan_bin, "skip")
    assert r.returncode == 66 and "data race" in r.stderr, r.stdout + r.stderr[-2000:]
