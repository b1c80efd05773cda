"""The oracle's C, and the library's host code, built with the address and
undefined-behaviour sanitizers (gcc/g++ -fsanitize=address,undefined) and
driven through their functions: no report, every call does what it should."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(HERE, "sanitize", "oracle_driver.c"), "-o", exe, "-lm"]
    subprocess.check_call(cmd)
    env = dict(os.environ)
    # a library preloaded into every process would otherwise precede the
    # sanitizer runtime, which it refuses by default
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not found")
def test_host_library_under_sanitizers(tmp_path):
    """The library's C-ABI sources built host-only with g++ under the same
    sanitizers, kernel launchers replaced by stubs (tests/sanitize/
    launch_stubs.cpp), and driven through configuration checks, sizing, index
    and window bookkeeping and argument errors (tests/sanitize/
    host_driver.cpp): no report, every expectation holds."""
    csrc = os.path.join(ROOT, "kv_cache_top_srht_amd", "csrc")
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + csrc,
           os.path.join(csrc, "pariskv_api.cpp"), os.path.join(csrc, "si_api.cpp"),
           os.path.join(HERE, "sanitize", "launch_stubs.cpp"),
           os.path.join(HERE, "sanitize", "host_driver.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.check_call(cmd)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
