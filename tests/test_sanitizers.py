"""Sanitizer builds of the CPU-side code, run in the CPU suite.

Two small drivers (tests/sanitize/) exercise the fp64 oracle (oracle/la_oracle.c,
with its worker threads) and the library's host-side logic
(linear_attention_amd/csrc/host_logic.h: argument checks, slopes, the
segment plan and its workspace size, the debug-mode metadata checks).  Each is
built with gcc/g++ under AddressSanitizer + UndefinedBehaviorSanitizer, and
the oracle also under ThreadSanitizer; any sanitizer report or failed check
fails the test.  Only host code is built here: no GPU code is instrumented.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ASAN_UBSAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build_and_run(cmd, exe, ok_line):
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    # verify_asan_link_order=0: the environment may preload a library ahead of
    # the ASan runtime; that is harmless for these drivers
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stderr
    assert r.returncode == 0 and ok_line in r.stdout, f"rc={r.returncode}\n{r.stdout}\n{report}"
    for marker in ("runtime error", "ERROR: AddressSanitizer", "WARNING: ThreadSanitizer", "LeakSanitizer"):
        assert marker not in report, report


@pytest.fixture(scope="module")
def compilers():
    for c in ("gcc", "g++"):
        if not shutil.which(c):
            pytest.skip(f"{c} not found")


def test_oracle_under_asan_ubsan(compilers, tmp_path):
    _build_and_run(["gcc", "-std=c11", *ASAN_UBSAN, os.path.join(ROOT, "oracle", "la_oracle.c"),
                    os.path.join(SAN, "oracle_driver.c"), "-lm", "-lpthread"],
                   str(tmp_path / "oracle_asan"), "oracle driver ok")


def test_oracle_threads_under_tsan(compilers, tmp_path):
    _build_and_run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=thread", os.path.join(ROOT, "oracle", "la_oracle.c"),
                    os.path.join(SAN, "oracle_driver.c"), "-lm", "-lpthread"],
                   str(tmp_path / "oracle_tsan"), "oracle driver ok")


def test_host_logic_under_asan_ubsan(compilers, tmp_path):
    _build_and_run(["g++", "-std=c++17", *ASAN_UBSAN, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "linear_attention_amd", "csrc"), os.path.join(SAN, "host_driver.cpp")],
                   str(tmp_path / "host_asan"), "host driver ok")
