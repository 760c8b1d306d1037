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
    src = os.path.join(ROOT, b.TRAFFIC_SOURCE["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for k in ("gate_up_gemm", "down_gemm"):
        want = b.TRAFFIC[k]["fetch_bytes"] + b.TRAFFIC[k]["write_bytes"]
        assert b.measured_traffic(k) == (want if sha == b.TRAFFIC_SOURCE["sha256"] else None)
    assert b.measured_traffic("combine") is None
    # any other source text: no traffic figure
    b.TRAFFIC_SOURCE = dict(b.TRAFFIC_SOURCE, sha256="0" * 64)
    assert b.measured_traffic() is None


def test_roofline_picks_the_higher_floor_and_keeps_both_fractions():
    b = _bench_module()
    # 1e12 flop and 1e10 bytes in 1 ms: MFMA floor 0.4 ms > HBM floor 1.25 ms? no:
    # HBM floor 1e10 / 8e12 = 1.25 ms, MFMA floor 1e12 / 2.5e15 = 0.4 ms -> hbm
    roof, mfma, hbm = b.gemm_roofline("gate_up_gemm", 1e12, 1e10, 2.0)
    assert roof["bound"] == "hbm" and roof["frac"] == hbm["frac"]
    assert roof["mfma_frac"] == mfma["frac"] == round(1e12 / 2e-3 / 1e12 / 2500.0, 4)
    roof, mfma, hbm = b.gemm_roofline("down_gemm", 1e13, 1e9, 10.0)
    assert roof["bound"] == "mfma" and roof["hbm_frac"] == hbm["frac"]


def test_side_modes_are_listed_in_the_help():
    """--copy-probe and --bmm-reference are separate modes (their own JSON
    line, no benchmark line); both must stay reachable from the command line."""
    out = subprocess.run([sys.executable, "bench.py", "--help"], capture_output=True, text=True,
                         cwd=ROOT, timeout=120)
    assert out.returncode == 0
    assert "--copy-probe" in out.stdout and "--bmm-reference" in out.stdout
