"""The oracle's pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake into a copy of oracle/sconv_oracle.c, builds
that copy, and runs tests/test_oracle_pins.py against it in a child process
(the oracle module loads the copy named by SCONV_ORACLE_LIB).  The pins must
fail.  A mutation that no pin notices would mean the oracle could be wrong
there without anything to show it.  Every planted mistake keeps each
memory access inside its buffer, so a failing run is a failing pin, not a
crash; and the unmutated copy, built and run the same way, must pass.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sconv_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# name, text as written in the oracle (must occur exactly once), mistake
MUTATIONS = [
    ("fused: taps reversed",
     "const int64_t lag = W - 1 - k;\n          const int64_t src = pos - lag;",
     "const int64_t lag = k;\n          const int64_t src = pos - lag;"),
    ("fused: same-forward test off by one",
     "} else if (t - lag >= q) {", "} else if (t - lag > q) {"),
    ("fused: stream offset missing from the tap read",
     "(src % N) * cs2 + off_s + j);", "(src % N) * cs2 + j);"),
    ("fused: logical block of the tap off by one",
     "const int64_t lblk = src / N;", "const int64_t lblk = (src + 1) / N;"),
    ("fused: weight columns reversed",
     "ld(w, dtype, c * w_sc + (int64_t)k * w_sk)",
     "ld(w, dtype, c * w_sc + (int64_t)(W - 1 - k) * w_sk)"),
    ("fused: residual inside the activation",
     "double y = activate(acc, act);",
     "double y = activate(acc + (residual ? ld(x, dtype, t * x_rs + c) : 0.0), act) -"
     " (residual ? ld(x, dtype, t * x_rs + c) : 0.0);"),
    ("fused: insert copies another head's input",
     "t * x_rs + (int64_t)h * ws + j, dtype);", "t * x_rs + j, dtype);"),
    ("bf16 rounding truncates",
     "double r = nearbyint(a / q) * q;", "double r = floor(a / q) * q;"),
    ("SiLU sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("metadata: request ranges closed at the end",
     "if ((int64_t)qsl[rr] <= t && t < (int64_t)qsl[rr + 1]) {",
     "if ((int64_t)qsl[rr] <= t && t <= (int64_t)qsl[rr + 1]) {"),
    ("metadata: padded rows not zero",
     "seq_idx_out[t] = 0;      /* padded rows are zero-filled */",
     "seq_idx_out[t] = num_reqs - 1;"),
    ("varlen: final state in reverse order",
     "const int64_t ui = L - S + m;", "const int64_t ui = L - 1 - m;"),
    ("varlen: bias dropped",
     "double acc = bias ? ld(bias, dtype, c) : 0.0;\n        for (int32_t k = 0; k < W; ++k) {\n"
     "          const int64_t ui = i - S + k;",
     "double acc = 0.0;\n        for (int32_t k = 0; k < W; ++k) {\n"
     "          const int64_t ui = i - S + k;"),
    ("update: state not shifted",
     "slot * ss_slot + (int64_t)c * ss_c + (int64_t)(m + 1) * ss_k, dtype);",
     "slot * ss_slot + (int64_t)c * ss_c + (int64_t)m * ss_k, dtype);"),
    ("multi-token update: shift state one entry late",
     "const int64_t j = seqlen + m;", "const int64_t j = seqlen + m - 1;"),
    ("ring update: tap column off by one",
     "v = ld(st_in, dtype, sbase + (pos % L) * ss_k);",
     "v = ld(st_in, dtype, sbase + ((pos + 1) % L) * ss_k);"),
    ("ring update: write column off by one",
     "copy_elem(st_out, sbase + ((s + i) % L) * ss_k,",
     "copy_elem(st_out, sbase + ((s + i + 1) % L) * ss_k,"),
    ("window gather: window one row late",
     "int64_t row = p - d_conv + k;", "int64_t row = p - d_conv + k + 1;"),
    ("window gather: rows before 0 mirrored, not clamped",
     "if (row < 0) row = 0;", "if (row < 0) row = -row;"),
    ("SSM-state gather: last live slot skipped",
     "for (int64_t i = 0; i < n; ++i) {\n    /* Slot i receives",
     "for (int64_t i = 0; i < n - 1; ++i) {\n    /* Slot i receives"),
    ("SSM-state gather: rows counted from the end",
     "copy_elem(out, i * out_rs + e, states, r * states_rs + e, dtype);",
     "copy_elem(out, i * out_rs + e, states, (num_chunks - 1 - r) * states_rs + e, dtype);"),
    ("threaded fused op: each range but the last drops its last row",
     "T * i / nthreads, T * (i + 1) / nthreads, ORC_OK};",
     "T * i / nthreads, T * (i + 1) / nthreads - (i + 1 < nthreads), ORC_OK};"),
]


def _run_pins(tmp, name, text):
    """Build `text` as the oracle in `tmp` and run the pins against it;
    returns the child's exit status and the tail of its output."""
    import oracle
    src = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"{name}.so")
    with open(src, "w") as f:
        f.write(text)
    # the header sits next to the source
    hdr = os.path.join(tmp, "sconv_oracle.h")
    if not os.path.exists(hdr):
        with open(os.path.join(ROOT, "oracle", "sconv_oracle.h")) as f, open(hdr, "w") as g:
            g.write(f.read())
    subprocess.run(oracle.compile_command(src, lib), check=True, capture_output=True)
    env = dict(os.environ, SCONV_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-600:]


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("mutants"))
    base = open(SRC).read()
    jobs = [("unmutated", base)]
    for k, (name, old, new) in enumerate(MUTATIONS):
        assert base.count(old) == 1, f"{name}: the text to mutate must occur once"
        jobs.append((f"m{k}", base.replace(old, new)))
    with ThreadPoolExecutor(max(1, min(4, os.cpu_count() or 1))) as ex:
        out = list(ex.map(lambda j: _run_pins(tmp, *j), jobs))
    return dict(zip([j[0] for j in jobs], out))


def test_unmutated_copy_passes_the_pins(results):
    rc, tail = results["unmutated"]
    assert rc == 0, tail


@pytest.mark.parametrize("k", range(len(MUTATIONS)), ids=[m[0] for m in MUTATIONS])
def test_pins_catch_the_mistake(results, k):
    rc, tail = results[f"m{k}"]
    assert rc == 1, f"{MUTATIONS[k][0]}: the pins did not fail (exit {rc}): {tail}"
