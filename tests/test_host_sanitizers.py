"""The host packers (asp_host.cpp, asp_svdq_host.cpp) built by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer next to a driver that calls
every host entry point on valid and invalid inputs (tests/host/): the run
must finish cleanly.  CPU only; the device code is not part of this build."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "wam_asp_w4a4_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_entry_points_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    build = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"),
             os.path.join(CSRC, "asp_host.cpp"), os.path.join(CSRC, "asp_svdq_host.cpp"),
             "-o", exe]
    b = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-2000:]
    # verify_asan_link_order=0: the environment may preload another library
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host entry points ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
