"""The host code (planner, policy, runner, the entry points' argument
checks) under AddressSanitizer and UndefinedBehaviorSanitizer: the C-ABI and
policy tests, run in a child process against the instrumented build of the
library (paged_gqa_decode_pkv_amd/sanitize.py).  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_code_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, "-m", "paged_gqa_decode_pkv_amd.sanitize"], cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
