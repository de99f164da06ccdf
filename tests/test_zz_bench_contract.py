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
    print("bench.py --steps 8 --warmup 2 --cpu-budget 0.3 (decode + prefill)", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "8",
                        "--warmup", "2", "--cpu-budget", "0.3"],
                       capture_output=True, text=True, timeout=170, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    assert j["unit"] == "tokens/s" and j["n_gpus"] == 1
    assert j["steps"] == 8 and j["warmup"] == 2
    assert j["higher_is_better"] is True and j["scaling"] == "weak"
    assert j["vs_baseline"] is None and j["data"] == "synthetic" and j["dtype"] == "bf16"
    assert j["config"]["workload"] == "batched_decode" and j["config"]["requests"] == 256
    assert j["value"] > 0 and j["ms_per_step"] > 0 and j["wall_ms_per_step"] >= j["ms_per_step"]
    # tokens/s over exactly the timed steps
    assert math.isclose(j["value"], 256 / (j["ms_per_step"] * 1e-3), rel_tol=1e-3)
    for part, nbytes in ((j, 3161224), (j["prefill"], None)):
        rf = part["roofline"]
        assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
        assert rf["achieved"] > 0 and math.isclose(rf["frac"], rf["achieved"] / rf["peak"],
                                                    abs_tol=1e-4)
        assert rf["traffic"] is None or rf["traffic"] > 0
        assert rf["frac_trace"] is None or 0 < rf["frac_trace"] < 1
        if nbytes:
            assert rf["bytes_per_launch"] == nbytes
        cpu = part["cpu_baseline"]
        assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
        assert cpu["unit"] == "tokens/s" and cpu["sample"] and cpu["cpu_model"]
        # the same algorithmic bytes per token as the GPU line
        per_token = rf["bytes_per_launch"] * (4 if part is j["prefill"] else 1) / (
            256 if part is j else part["config"]["non_pad_tokens"])
        assert math.isclose(cpu["GBs"], cpu["value"] * per_token / 1e9, rel_tol=1e-2, abs_tol=2e-3)
        if cpu["cores"] > 1:
            assert cpu["single_thread"]["value"] > 0
    m = j["machine"]  # the probe kernels are built with the library
    assert 1.0 < m["copy_TBs"] < 8.0 and 1.0 < m["prefill_pattern_TBs"] < 8.0
    assert 1.0 < m["prefill_pattern_at_launch_size_TBs"] < 8.0
    assert 1.0 < m["prefill_layout_with_taps_and_halo_TBs"] < m["prefill_layout_TBs"] < 8.0
    # the prefill's ceiling is the best of the machine's figures for its traffic
    assert math.isclose(j["prefill"]["roofline"]["ceiling_GBs"],
                        1e3 * max(m["prefill_pattern_TBs"], m["prefill_pattern_at_launch_size_TBs"],
                                  m["prefill_layout_TBs"]), rel_tol=1e-3)
    assert 0 < m["empty_launch_us"] < m["decode_chain_floor_us"]
    assert 0 < m["empty_launch_us"] < m["decode_chain_floor_us_args_loaded"]
    assert math.isclose(j["roofline"]["launch_over_floor"],
                        j["roofline"]["launch_us"] / m["decode_chain_floor_us"], rel_tol=1e-2)
    assert j["prefill"]["roofline"]["frac_of_ceiling"] > 0
    p = j["prefill"]
    assert p["workload"] == "mixed_prefill" and p["steps"] == 8 and p["warmup"] == 2
    assert p["config"]["streams"] == 4 and p["value"] > 0
    assert math.isclose(p["value"], p["config"]["non_pad_tokens"] / (p["ms_per_step"] * 1e-3),
                        rel_tol=1e-3)
