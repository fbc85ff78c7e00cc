"""Entry points called from several host threads at once, each on its own stream.

The library keeps per-device caches (CU count, occupancy per kernel, fa2_bwd_noalloc's scratch
address) that the first calls fill, and a thread-local error string. `threads_child.py` runs in
a fresh process so that ten threads' first calls coincide; every thread's results must equal,
bit for bit, the same calls repeated afterwards on one thread.
"""
import os
import subprocess
import sys

import pytest

from tests.gpu_helpers import announce, device

pytestmark = pytest.mark.gpu


def test_concurrent_host_threads():
    device()
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "threads_child.py")
    announce("entry points from 10 host threads at once (child process)")
    r = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True, timeout=240)
    print(r.stdout[-4000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0, f"child exited {r.returncode}"
    assert "ALL OK" in r.stdout
