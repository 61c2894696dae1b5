"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_oracle_main.c compresses small seeded matrices with every coding,
route and several precisions (and the per-row refinement), decodes them to every
output kind, and decodes damaged copies with per-tile status.  Built here with
gcc and the host sanitizers; any out-of-bounds access, leak or undefined
operation aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
SOURCES = [os.path.join(ORACLE, f) for f in ("epo_codec.c", "epo_convert.c", "epo_lattice.c", "epo_rans.c")]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_memory_and_ub_safe_on_intact_and_damaged_streams(tmp_path):
    exe = str(tmp_path / "sanitize_oracle")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           "-I", ORACLE] + SOURCES + [os.path.join(ROOT, "tests", "sanitize_oracle_main.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr
