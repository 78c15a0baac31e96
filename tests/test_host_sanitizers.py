"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The calibration (the library's only host-side arithmetic) is compiled with
g++ -fsanitize=address,undefined together with a driver that exercises it
over several sizes and its argument checks; any sanitizer report fails the
run (halt_on_error)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_calibrate_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "calibrate_asan"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "sparse_attention_decode_loki_amd", "csrc", "calibrate.cpp"),
           os.path.join(ROOT, "tests", "host", "calibrate_asan_main.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
