"""The host half of the library (codec construction in host_codec.cpp) built
with AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU over
the shapes the library accepts (tests/host_check.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_codec_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", os.path.join(ROOT, "tests", "host_check.cpp"),
           os.path.join(ROOT, "kv_cache_compression_tq_amd", "csrc", "host_codec.cpp"), "-lpthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
