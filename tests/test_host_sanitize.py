"""The file stager's host logic (its only multi-threaded code) under ThreadSanitizer
and AddressSanitizer: filestage.hip is built with the host compiler against a stub
HIP runtime (tests/host_stub: copies and event records run later on a per-stream
thread, as on a DMA engine) and driven through concurrent consumers, buffer reuse, a
failed read, the rate cap, an empty call and destruction with queued work.  A buffer
reused before its copy ran, a job freed under a worker, or any other race or invalid
access fails the run.  No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "lossy_kv_draft_amd", "csrc", "filestage.hip")
DRIVER = os.path.join(ROOT, "tests", "host_stub", "stager_driver.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host C++ compiler")
@pytest.mark.parametrize("san", ["thread", "address,undefined"])
def test_file_stager_host_paths_under_sanitizer(san, tmp_path):
    exe = str(tmp_path / "stager")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={san}",
           "-I", os.path.join(ROOT, "tests", "host_stub"), "-x", "c++", SRC, "-x", "none", DRIVER, "-o", exe,
           "-lpthread"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "stager host paths ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
