"""The host-side bookkeeping and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/host_fuzz.cpp links the library's host sources (pool,
sequences, prefix cache, swap, scheduler) and the oracle's C source, built
here with g++/gcc and -fsanitize=address,undefined, and drives them with
random operations for several seeds, checking the pool's accounting after
every operation.  Any memory error, undefined behaviour or failed check
ends the run with a non-zero status.  No GPU code is built or run.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_indirected_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitize")
    obj = str(d / "oracle.o")
    exe = str(d / "host_fuzz")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", *SAN, "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", obj], check=True)
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "sanitize", "host_fuzz.cpp"),
                    *[os.path.join(CSRC, f) for f in ("errors.cpp", "pool.cpp", "sched.cpp")],
                    obj, "-fopenmp", "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_random_operations_clean_under_sanitizers(fuzz_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([fuzz_exe, str(seed), "2500"], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    words = r.stdout.split()
    assert words[:2] == ["ok", "seed"], r.stdout
    # every kind of operation succeeded at least once, and copy-on-write
    # copies were handed out
    counts = [int(x) for x in words[4:16]]
    assert len(counts) == 12 and min(counts) > 0, r.stdout
    assert int(words[-1]) > 0, r.stdout
