"""bench.py's command line on the CPU: a request for several GPUs is refused
with a message and no JSON line (the library has no multi-GPU path)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bad_step_counts_are_refused():
    for argv in (["--steps", "0"], ["--warmup", "-1"], ["--requests", "0"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                           capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, argv
        assert "must be" in r.stderr and r.stdout.strip() == ""
