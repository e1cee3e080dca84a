"""The debug build (libpkv_debug.so, PKV_DEBUG): device preconditions that
the release build only tolerates are reported as PKV_EINVAL, and valid calls
give bit for bit the release build's results.

The debug library is loaded by a child process (the package picks it when
PKV_DEBUG=1), which runs debug_cases.py; this process runs the same valid
calls on the release library and compares the saved outputs.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import debug_cases
import paged_kv_cache_indirected_amd as pkv
from harness import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_debug_build_reports_violations_and_matches_release_bitwise(tmp_path):
    assert os.path.basename(pkv.LIB_PATH) == "libpkv.so"
    say("[debug] valid calls on the release library")
    rel = debug_cases.valid_outputs()
    env = dict(os.environ, PKV_DEBUG="1")
    say("[debug] child process on libpkv_debug.so")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_cases.py"),
                        str(tmp_path)], env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout[-6000:])
    print(r.stderr[-6000:], file=sys.stderr)
    assert r.returncode == 0, r.stderr[-2000:]
    dbg = np.load(os.path.join(tmp_path, "valid.npz"))
    assert sorted(dbg.files) == sorted(rel)
    for name, bits in rel.items():
        assert np.array_equal(bits, dbg[name]), name
