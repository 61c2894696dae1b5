"""The multithreaded host compressor under the host sanitizers.

tests/sanitize_host_encoder_main.cpp compresses small seeded matrices (several
rates, the three routes) with 1 and 4 worker threads and requires identical
containers.  It is built twice with g++: with AddressSanitizer and
UndefinedBehaviorSanitizer (out-of-bounds accesses, leaks, undefined
operations) and with ThreadSanitizer (data races between the workers).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "dit_weight_compression_amd", "csrc", "ep_encode.cpp"),
           os.path.join(ROOT, "tests", "sanitize_host_encoder_main.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
@pytest.mark.parametrize("sanitizers", ["address,undefined", "thread"])
def test_host_encoder_sanitized_and_thread_count_invariant(tmp_path, sanitizers):
    exe = str(tmp_path / "sanitize_host_encoder")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={sanitizers}",
           "-pthread", "-ffp-contract=off", "-I", os.path.join(ROOT, "include")] + SOURCES + ["-o", exe]
    if sanitizers != "thread":
        cmd.insert(6, "-fno-sanitize-recover=all")
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr
    assert "WARNING: ThreadSanitizer" not in r.stderr
