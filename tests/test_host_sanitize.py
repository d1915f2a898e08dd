"""The host half of libfm (plan builder, C ABI) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer (device functions stubbed),
then driven over a grid of configurations and invalid arguments: any invalid
memory access, leak or undefined operation fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "stft_mel_spectrogram_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_plan_builder_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "fm_host_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fm_plan.cpp"), os.path.join(CSRC, "fm_api.cpp"),
           os.path.join(HERE, "device_stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
