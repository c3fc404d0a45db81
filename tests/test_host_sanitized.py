"""The library's host code (metadata, packer, tile builder, error text) built with AddressSanitizer and
UndefinedBehaviorSanitizer by the host compiler and driven through valid and invalid arguments
(tests/native/host_driver.cpp).  CPU only; the device code is not part of this build."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{ROOT}/include", f"-I{ROOT}/position_agnostic_paged_amd/csrc",
           os.path.join(ROOT, "tests", "native", "host_driver.cpp"),
           os.path.join(ROOT, "position_agnostic_paged_amd", "csrc", "host.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
