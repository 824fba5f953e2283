"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
runs its pins clean (learned_kv_chunk_amd/sanitize.py, oracle part; the HIP
library's host-side run, which rebuilds every kernel, is run by hand:
python -m learned_kv_chunk_amd.sanitize)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, "-m", "learned_kv_chunk_amd.sanitize", "--skip-hip"],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "sanitizer runs clean" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
