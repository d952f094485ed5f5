"""The library's calls are re-entrant: its per-device host state (CU count,
large-LDS kernel attributes, launch plans) is initialised once, thread-safely.
The first GEMV and skinny calls of a fresh process, made from 4 threads on
separate streams, must each match the oracle."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_first_calls_from_four_threads():
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "concurrent_first_calls.py")],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": ok") == 4, r.stdout
