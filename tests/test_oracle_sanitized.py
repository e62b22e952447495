"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): oracle/sanitize_main.c drives every entry point over small
inputs that reach the edge paths for the three cache types; any invalid
memory access or undefined behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_oracle_runs_clean_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ORACLE, "mla_oracle.c"), os.path.join(ORACLE, "sanitize_main.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle sanitizer run: ok" in res.stdout
    assert "runtime error" not in res.stderr, res.stderr
