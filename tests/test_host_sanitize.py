"""The host layer of liborbq (api.cpp, codebook.cpp) built for the CPU with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, its GPU launchers replaced by stubs that abort
(tests/host_sanitize/stubs.cpp), and driven through the C ABI's host-only paths
(tests/host_sanitize/driver.cpp): the Lloyd-Max builder for d = 3 .. 12288 and 1 .. 8 bits (1 .. 6 above d = 256), the
validators, the size helpers and every entry point's argument checks."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE), reason="needs g++ and the HIP headers")
def test_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "orbq_host_driver")
    csrc = os.path.join(ROOT, "calibration_free_w4a4_amd", "csrc")
    here = os.path.join(ROOT, "tests", "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}",
           "-x", "c++", os.path.join(csrc, "api.cpp"), os.path.join(csrc, "codebook.cpp"),
           os.path.join(here, "stubs.cpp"), os.path.join(here, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert r.stdout.strip().startswith("ok "), r.stdout[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
