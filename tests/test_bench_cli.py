"""bench.py's command-line contract on the host: the layer is measured on one
GPU, so a request for several exits at once with a message and status 2,
before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == ""          # no JSON line
