"""The host core (csrc/host.cpp, csrc/pool.cpp: plain C++ with no HIP)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
driven through every host entry point by tests/host_sanitize.cpp, with
exactly sized buffers (CPU only)."""
import os
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(REPO, "heterogeneous_adapter_batching_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_core_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "host_sanitize"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
    subprocess.run(["g++", *flags, "-I", os.path.join(REPO, "include"), "-I", CSRC,
                    os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "pool.cpp"),
                    os.path.join(REPO, "tests", "host_sanitize.cpp"), "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host core ok" in r.stdout
