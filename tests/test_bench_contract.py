"""The benchmark's host-side contract, without a GPU: more than one GPU is
refused before anything touches a device, and the HBM traffic figure is taken
from a committed counter summary only when that summary was made on the
current kernel source."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_needs_the_current_kernel_source(tmp_path):
    bench = load_bench()
    sha = bench.kernel_sha()
    assert len(sha) == 16
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = "kernel_sha256_16: %s\ntraffic_bytes_per_launch: 144000000\n"
    (prof / "cur.txt").write_text(body % sha)
    (prof / "old.txt").write_text(body % ("0" * 16))
    (prof / "bad.txt").write_text("kernel_sha256_16: %s\n" % sha)
    bench.ROOT = str(tmp_path)
    assert bench.read_traffic("cur.txt", 1.0) == 144000000.0
    assert bench.read_traffic("old.txt", 1.0) is None
    assert bench.read_traffic("bad.txt", 1.0) is None
    assert bench.read_traffic("missing.txt", 1.0) is None
