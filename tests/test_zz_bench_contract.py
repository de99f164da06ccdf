"""One short run of bench.py with its defaults (the batched decode step) in a
child process, and the keys and types of the JSON line it prints.  Named to
be collected last: it starts a second process on the GPU."""
from __future__ import annotations

import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_default_bench_line():
    print("bench.py --steps 8 --warmup 2 --cpu-budget 0.3 (batched decode)", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "8",
                        "--warmup", "2", "--cpu-budget", "0.3"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    assert j["unit"] == "tokens/s" and j["n_gpus"] == 1
    assert j["steps"] == 8 and j["warmup"] == 2
    assert j["higher_is_better"] is True and j["scaling"] == "weak"
    assert j["vs_baseline"] is None and j["data"] == "synthetic" and j["dtype"] == "bf16"
    assert j["config"]["workload"] == "batched_decode" and j["config"]["requests"] == 256
    assert j["value"] > 0 and j["ms_per_step"] > 0
    # tokens/s over exactly the timed steps
    assert math.isclose(j["value"], 256 / (j["ms_per_step"] * 1e-3), rel_tol=1e-3)
    rf = j["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and math.isclose(rf["frac"], rf["achieved"] / rf["peak"],
                                                abs_tol=1e-4)
    assert rf["traffic"] is None or rf["traffic"] > 0
    assert rf["bytes_per_launch"] == 3161224
    cpu = j["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0
    assert cpu["unit"] == "tokens/s" and cpu["sample"]
