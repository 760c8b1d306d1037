"""bench.py's command-line contract that needs no GPU: a request for more
than one GPU is refused with a message and exit status 2, before any device
work; the roofline traffic figure is reported only for the kernel source it
was measured on."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_traffic_only_for_the_measured_source(tmp_path):
    b = _bench_module()
    src = os.path.join(ROOT, b.GATE_UP_TRAFFIC["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    want = b.GATE_UP_TRAFFIC["fetch_bytes"] + b.GATE_UP_TRAFFIC["write_bytes"]
    assert b.measured_traffic() == (want if sha == b.GATE_UP_TRAFFIC["sha256"] else None)
    # any other source text: no traffic figure
    b.GATE_UP_TRAFFIC = dict(b.GATE_UP_TRAFFIC, sha256="0" * 64)
    assert b.measured_traffic() is None
