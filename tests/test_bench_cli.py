"""bench.py's command-line contract on the host: one GPU only."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout == ""  # no JSON line
