"""bench.py's command-line contract on the host: one GPU only, and probe rows
checked before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "no multi-GPU path" in r.stderr


def test_unknown_traffic_row_is_refused_before_gpu_work():
    r = _run("--traffic-probe", "--traffic-row", "no_such_row")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr
