"""The host encoder and blob validator built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, host code only) and run over every format,
several geometries, constant and one-rare-symbol layers, short buffers and
corrupted blobs (tests/sanitize/host_driver.cpp)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_encoder_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(ROOT, "decode_gemm_tile_amd", "csrc", "dgt_host.cpp"),
           "-lpthread", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.startswith("ok:"), r.stdout
