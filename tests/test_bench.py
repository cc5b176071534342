"""bench.py's host-side contract (no GPU needed): more than one GPU is
refused with a one-line JSON message and a non-zero exit, before anything
touches a device."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    msg = json.loads(lines[0])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
