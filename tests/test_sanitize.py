"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer) of the
host-only half of libmoshi.so (config validation, weight count, slot table,
frame and forced-token validation: csrc/host.h) and of the test oracle, each
driven through all of its entry points by a small C/C++ program under
tests/sanitize/. Any sanitizer report aborts the program and fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
ENV.pop("LD_PRELOAD", None)


def _run(cmd, exe):
    subprocess.check_call(cmd)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_logic_sanitized(tmp_path):
    exe = str(tmp_path / "host_check")
    out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                "-I", os.path.join(ROOT, "full_duplex_speech_amd", "csrc"),
                os.path.join(HERE, "host_check.cpp"), "-o", exe], exe)
    assert "host checks ok" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_check")
    out = _run(["gcc", "-std=c11", *SAN, os.path.join(HERE, "oracle_check.c"), "-o", exe, "-lm"],
               exe)
    assert "oracle checks ok" in out
