"""Build libsconv.so in-tree with hipcc for gfx950.

    python -m depthwise_causal_conv1d_amd.build [--define NAME=VALUE ...] [--out PATH]

Every HIP source under csrc/ plus the host status unit is compiled into one
shared library next to this file.  Packed-fp32 instructions are disabled on
purpose (the compiler would otherwise form v_pk_* FP32 ops from plain float
code).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsconv.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsconv)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "status.cpp")]


def flags(defines=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # leading scalar kernel arguments preloaded into SGPRs by the
            # hardware (the fused kernel's first-hop values)
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-I", os.path.join(HERE, "..", "include"), *[f"-D{d}" for d in defines]]


def command(out: str):
    """The whole build as one hipcc command (for reference)."""
    return [hipcc(), *flags(), "-shared", "-o", out, *sources()]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source to an object in parallel, then link the shared
    library.  `defines` are -D switches (the tuning knobs of csrc/; the
    defaults are the measured choices)."""
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = out + ".objs%d" % os.getpid()
    os.makedirs(tmpdir, exist_ok=True)
    try:
        srcs = sources()
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[hipcc(), *flags(defines), "-c", "-o", o, src] for src, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = min(len(cmds), max(1, min(os.cpu_count() or 1, 16)))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True),
                                  cmds))
        for c, res in zip(cmds, results):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed on " + c[-1])
        tmp = out + ".tmp%d" % os.getpid()
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libsconv.so")
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libsconv.so for gfx950")
    ap.add_argument("--define", "-D", action="append", default=[],
                    help="a tuning switch of csrc/ (NAME=VALUE), e.g. SCONV_FUSED_MS_ORDER=2; "
                         "the defaults are the measured choices")
    ap.add_argument("--out", default=LIB, help="where to write the library (default: in-tree)")
    a = ap.parse_args()
    print(build(verbose=True, out=a.out, defines=a.define))
