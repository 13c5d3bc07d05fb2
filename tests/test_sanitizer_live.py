"""Under tests/sanitize.sh (KVC_SANITIZE=1) the oracle runs instrumented: a
child process that hands orc_encode_stream an output buffer smaller than the
capacity it states must be stopped by AddressSanitizer.  Skipped otherwise."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.skipif(os.environ.get("KVC_SANITIZE") != "1", reason="sanitizer run only")

CHILD = r"""
import numpy as np, oracle
lib = oracle._load()
q = np.full(512, 5, np.uint8)
rows = np.tile(np.arange(0, 64 * 1024, 1024, dtype=np.uint16)[:64], (512, 1))  # flat rows: ~6 bits/symbol
out = np.zeros(8, np.uint8)  # far fewer bytes than the stated capacity
lib.orc_encode_stream(q.ctypes.data, 512, 64, rows.ctypes.data, out.ctypes.data, 4096)
print("not caught")
"""


def test_out_of_bounds_write_is_caught():
    r = subprocess.run([sys.executable, "-c", CHILD], env=dict(os.environ), capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0, r.stdout
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr
