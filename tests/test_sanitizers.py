"""The CPU suite once more against AddressSanitizer + UndefinedBehaviorSanitizer
builds of the host code (the C-ABI library's host side, the oracle and the
input generator): see tests/sanitize.py.  Any sanitiser report aborts the
child run and fails this test."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(900)
def test_cpu_suite_clean_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize.py")], capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
