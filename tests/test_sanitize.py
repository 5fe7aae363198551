"""The oracle and the input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only), running the whole oracle chain
on small problems (oracle/sanitize_check.c).  Any out-of-bounds access, leak or
undefined operation aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "sanitize_check.c"), os.path.join(ROOT, "oracle", "oomb_oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": ok") == 4, r.stdout
    assert "runtime error" not in r.stderr, r.stderr
