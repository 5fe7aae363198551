"""Host code under sanitizers (gcc/g++, host code only, no GPU):
- the oracle and the input generator with AddressSanitizer and
  UndefinedBehaviorSanitizer, running the whole oracle chain on small problems
  (oracle/sanitize_check.c);
- the library's host-only code (paged_sparse_attention_amd/csrc/host.cpp) with
  ASan + UBSan and, for its threaded gradient add, ThreadSanitizer
  (tests/host_sanitize.cpp).
Any out-of-bounds access, leak, undefined operation or data race aborts the
run."""
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


CSRC = os.path.join(ROOT, "paged_sparse_attention_amd", "csrc")


def _host_driver(tmp_path, name, sanitize, env_extra):
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread", f"-fsanitize={sanitize}",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_sanitize.cpp"), os.path.join(CSRC, "host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(os.environ, **env_extra), timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validation: " in r.stdout and r.stdout.count(": ok") == 2, r.stdout
    assert "runtime error" not in r.stderr and "WARNING: ThreadSanitizer" not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    """The library's host-only code (csrc/host.cpp: descriptor validation and
    the threaded host-side gradient add) under AddressSanitizer and UBSan."""
    _host_driver(tmp_path, "host_asan", "address,undefined",
                 {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1"})


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_library_host_code_under_tsan(tmp_path):
    """The threaded host-side gradient add under ThreadSanitizer: the threads
    write disjoint blocks, so no data race may be reported."""
    _host_driver(tmp_path, "host_tsan", "thread", {"TSAN_OPTIONS": "halt_on_error=1"})
