"""The oracle's C built with the address and undefined-behaviour sanitizers
(gcc -fsanitize=address,undefined), driven through every function on seeded
inputs (tests/sanitize/oracle_driver.c): no report, every call succeeds."""
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
