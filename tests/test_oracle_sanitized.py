"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only):
tests/c/oracle_sanitize.c runs every oracle function over edge-case shapes on buffers of exactly
the documented sizes; any access outside them, or any undefined behaviour, fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed")
def test_oracle_is_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
           "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all calls clean" in r.stdout
