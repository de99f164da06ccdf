"""Benchmark of the paged short-convolution hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --probe          (machine ceilings, one JSON line)

Default (the headline): batched decode -- 256 requests x 1 token, history
lengths uniform in [1, 4096], H=32, D=128, ws=32 (C=1024), W=4, N=16, bf16,
SiLU and residual; one step is one launch of sconv_fused_insert_conv_qsl
(request search, insert and conv) replayed from a hipGraph.  The same line
carries a `prefill` object for the mixed varlen prefill -- 16 requests,
~20k rows, four streams of C=4096 over one shared cache, 10% PAD rows; one
step is sconv_seq_metadata + four sconv_fused_insert_conv launches -- so
that one run measures the metric's decode and prefill halves.

`--workload NAME` prints one line for one workload instead:
  batched_decode    the headline decode step alone
  decode_layer      the decode batch with all four streams of a layer
                    (ws=32 each) in one sconv_fused_insert_conv_streams launch
  mixed_prefill     the prefill step alone
  spec_decode       512 requests x 4 draft rows, C=4096, N=32; step = the
                    folded conv and the conv-window gather in one launch
                    (sconv_fused_insert_conv_gather; --gather-launch separate:
                    two), each replica with its own device-side real_count
                    uniform in [0, 512]
  ssm_prefill       8 x 4096 tokens, dim 8192, channel-major, state pool of
                    1024 slots; step = causal_conv1d_varlen_fwd
  ssm_decode        8 rows x dim 8192 against the same pool; step =
                    causal_conv1d_update
  ssm_spec_decode   8 rows x 4 draft tokens x dim 8192, ring states; step =
                    causal_conv1d_update_tokens
  ssm_state_gather  96 live of 128 slots, 2 MiB fp32 state rows; step =
                    gather_intermediate_ssm_state (device real_count)

Successive steps cycle through independent replicas of the workload's
inputs (own inputs, outputs, tables and cache blocks) so that at least
~512 MB separate two visits of the same bytes: every step reads HBM, not the
L2s or the 256 MB MALL.

Timing.  The library's code is loaded first (sconv_init), then the timed
steps, the warm-up steps and the dominant kernel alone are captured into
hipGraphs and uploaded; nothing runs before the warm-up.  Exactly W warm-up
steps run, then exactly K timed steps, bracketed by device synchronizations.
HIP events on the stream the steps run on bracket the K steps; a spin
kernel queued ahead of the first event keeps the host's graph submission
out of the interval.  `ms_per_step` and `value` (tokens per second) come
from those events; `wall_ms_per_step` is the host clock around the same
region, submission included.

`roofline` describes the workload's dominant kernel: algorithmic bytes per
launch divided by its average launch duration.  `frac` takes the duration
from HIP events around replays of a graph holding only that kernel (the
headline figure); `frac_trace` takes it from the committed rocprofv3 kernel
trace of the same command (profiles/), where tracing adds its own handling
to every dispatch, and is null once the kernel sources have changed since.
`cpu_baseline` times the oracle on a bounded sample of the same workload,
on every host core the process may use (rows or channels split across
threads) and single-threaded.  The default line's `machine` object gives
what the same GPU reaches, in the same run, on the reference kernels of
bench_probes.hip: the copy and the prefill's write patterns (TB/s) and
the decode kernel's dependent chain at its launch shape (us).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s and achieved HBM GB/s (% of peak) for fused paged sconv, decode + prefill"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "depthwise_causal_conv1d_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
FLUSH_BYTES = 512 << 20   # bytes that must separate two visits of a replica


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _strip_comments(text: str) -> str:
    """C/C++ source without its comments, blank lines and trailing blanks
    (none of these sources has a comment marker inside a string literal)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def _kernel_sources(kernel: str):
    """The csrc/ files a kernel is built from: the source that defines it
    and the headers it includes, transitively."""
    first = None
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip"):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                if re.search(r"\bvoid\s+" + re.escape(kernel) + r"\s*\(", f.read()):
                    first = name
                    break
    if first is None:
        raise KeyError(f"no source in {CSRC} defines {kernel}")
    seen, todo = [], [first]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.append(name)
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            for inc in re.findall(r'#include\s+"([^"/]+)"', f.read()):
                if os.path.exists(os.path.join(CSRC, inc)):
                    todo.append(inc)
    return sorted(seen)


def kernel_source_digest(kernel: str = None) -> str:
    """Hash of GPU sources without their comments, to tell whether stored
    traces and counters were taken on the kernels as they are now: of the
    files `kernel` is built from, or (no kernel) of every source."""
    names = sorted(os.listdir(CSRC)) if kernel is None else _kernel_sources(kernel)
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the kernel's current
    sources."""
    path = os.path.join(PROFILES, f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_sources:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest(kernel):
        return None
    return float(t.group(1))


def stored_trace(kernel: str, workload: str):
    """Average duration (us) of the dominant kernel in the committed
    rocprofv3 kernel-trace summary, if it was taken on the kernel's current
    sources."""
    path = os.path.join(PROFILES, f"{kernel.replace('_kernel', '')}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_sources:\s*([0-9a-f]+)", text)
    t = re.search(r"trace_avg_us:\s*([0-9.]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest(kernel):
        return None
    return float(t.group(1))


# ---------------------------------------------------------------- host facts

def cpu_threads() -> int:
    """Host threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when set (the share of a shared host it is given)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(n, 256))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- accounting

def fused_algorithmic_bytes(case, rows=None) -> int:
    """Bytes one fused launch over `rows` of case must move: input rows read
    (each once), distinct pre-forward cache positions tapped, slot writes and
    output writes of non-PAD rows, the weights, 24 B of per-row metadata and
    the block-table entries followed."""
    e = case.x.element_size()
    C, W, N = case.C, case.W, case.block_size
    pos = case.positions.numpy()
    sm = case.slot_mapping.numpy()
    qsl = case.query_start_loc.numpy()
    lo, hi = rows if rows is not None else (0, case.T)
    live = sm[lo:hi] >= 0
    n_live = int(live.sum())
    need = live.copy()
    before = set()  # rows ahead of the range read as same-forward taps
    taps = 0
    bt_entries = 0
    for r in range(case.num_reqs):
        a, b = max(int(qsl[r]), lo), min(int(qsl[r + 1]), hi)
        if a >= b:
            continue
        first = int(pos[int(qsl[r])])
        tapped = set()
        for t in range(a, b):
            if sm[t] < 0:
                continue
            for lag in range(1, W):
                src = int(pos[t]) - lag
                if src < 0:
                    continue
                if t - lag >= int(qsl[r]):
                    if t - lag >= lo:
                        need[t - lag - lo] = True
                    else:
                        before.add(t - lag)
                elif src < first:
                    tapped.add(src)
        taps += len(tapped)
        bt_entries += len({p // N for p in tapped})
    x_rows = int(need.sum()) + len(before)
    return (x_rows + taps + 2 * n_live) * C * e + C * W * e + 24 * (hi - lo) + 4 * bt_entries


def fused_streams_algorithmic_bytes(cases, rows=None) -> int:
    """Bytes one multi-stream launch must move: every stream's own bytes
    (fused_algorithmic_bytes), with the per-row metadata and the block-table
    entries, which the streams share, counted once."""
    c0 = cases[0]
    lo, hi = rows if rows is not None else (0, c0.T)
    shared = 24 * (hi - lo) + _bt_bytes(c0, rows)
    return sum(fused_algorithmic_bytes(c, rows) for c in cases) - (len(cases) - 1) * shared


def _bt_bytes(case, rows=None) -> int:
    """4 bytes per block-table entry the taps follow (as in
    fused_algorithmic_bytes)."""
    W, N = case.W, case.block_size
    pos = case.positions.numpy()
    sm = case.slot_mapping.numpy()
    qsl = case.query_start_loc.numpy()
    lo, hi = rows if rows is not None else (0, case.T)
    n = 0
    for r in range(case.num_reqs):
        a, b = max(int(qsl[r]), lo), min(int(qsl[r + 1]), hi)
        if a >= b:
            continue
        first = int(pos[int(qsl[r])])
        tapped = set()
        for t in range(a, b):
            if sm[t] < 0:
                continue
            for lag in range(1, W):
                src = int(pos[t]) - lag
                if src >= 0 and t - lag < int(qsl[r]) and src < first:
                    tapped.add(src)
        n += len({p // N for p in tapped})
    return 4 * n


def sub_case(case, rows, reqs, poison=None):
    """The requests `reqs` (rows `rows`) of a multi-batch case as a case of
    their own, for the oracle."""
    return case.select(rows, reqs)


def repeat_until(budget, once):
    """Oracle timing loop of the CPU baseline: call once(n) for n = 0, 1, ...
    (each call returns the tokens it covered and the seconds it took) until
    `budget` seconds of oracle time are spent, at least once.  Returns
    (tokens, seconds, calls)."""
    tokens, spent, n = 0, 0.0, 0
    while n == 0 or spent < budget:
        u, t = once(n)
        tokens += u
        spent += t
        n += 1
    return tokens, spent, n


def time_oracle_fused(case, activation="silu", threads=1):
    """Seconds the oracle spends on one fused launch of `case` (compact
    cache), its rows split over `threads` host threads.  The timed call
    includes its own marshalling: a copy of the compact cache it writes
    into."""
    import oracle
    from tests.helpers import to_np
    cache, bt, sm = case.compact()
    si, qs = oracle.seq_metadata(to_np(case.query_start_loc), case.num_reqs, case.num_actual,
                                 case.T)
    args = (to_np(case.x), to_np(case.weight), to_np(cache), to_np(case.positions), to_np(bt),
            si, to_np(sm), qs, case.off_s, case.ws, case.block_size, activation,
            case.use_residual)
    t0 = time.perf_counter()
    oracle.fused_insert_conv(*args, threads=threads)
    return time.perf_counter() - t0


# ---------------------------------------------------------------- workloads

class Workload:
    kernel_name = "fused_insert_conv_kernel"
    bound = "hbm"
    dtype = "bf16"
    unit = "tokens/s"     # of `value`: units of tokens_per_step per second
    oracle_split = True   # the oracle op of its CPU baseline has a threaded form

    def kernel(self, i):          # the dominant kernel alone
        raise NotImplementedError

    def kernels_per_call(self):   # launches of it per kernel(i)
        return 1

    def step_is_kernel(self):     # a step is one launch of the kernel, nothing more
        return self.step == self.kernel


class DecodeBench(Workload):
    """R independent decode batches of B requests sharing one large cache."""

    def __init__(self, dev="cuda", requests: int = 256, fold: bool = False):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        self.fold = fold
        self.B = B = requests
        per_batch = B * 12_350  # ~algorithmic bytes of one batch (exact value below)
        self.R = max(2, -(-FLUSH_BYTES // per_batch) + 16 * (B <= 256))
        t = time.time()
        self.case = workloads.batched_decode(device=dev, num_reqs=B * self.R,
                                             pool_blocks=int(B * self.R * 2 * 1.25) + 1)
        c = self.case
        log(f"batched_decode: {self.R} batches of {B} in {time.time() - t:.1f}s, cache "
            f"{c.cache.numel() * c.cache.element_size() / 2**30:.1f} GiB")
        self.x, self.w, self.cache = c.x.to(dev), c.weight.to(dev), c.cache
        self.pos, self.sm, self.bt = c.positions.to(dev), c.slot_mapping.to(dev), c.block_table.to(dev)
        self.out = torch.empty_like(self.x)
        self.qsl = torch.arange(B + 1, dtype=torch.int32, device=dev)
        self.si = torch.empty(B, dtype=torch.int32, device=dev)
        self.qs = torch.empty(B, dtype=torch.int32, device=dev)
        self.bytes_per_launch = fused_algorithmic_bytes(c, (0, B))
        self.tokens_per_step = B

    def rows(self, i):
        return slice(i * self.B, (i + 1) * self.B)

    def kernel(self, i):
        s, c = self.rows(i), self.case
        if self.fold:
            self.lib.sconv_fused_insert_conv_qsl(self.x[s], self.w, self.cache, self.pos[s],
                                                 self.bt[s], self.qsl, self.B, self.sm[s],
                                                 c.off_s, c.ws, c.block_size, "silu", True,
                                                 out=self.out[s])
            return
        self.lib.sconv_fused_insert_conv(self.x[s], self.w, self.cache, self.pos[s], self.bt[s],
                                         self.si, self.sm[s], self.qs, c.off_s, c.ws,
                                         c.block_size, "silu", True, out=self.out[s])

    def step(self, i):
        if not self.fold:
            self.lib.sconv_seq_metadata(self.qsl, self.B, self.B, self.si, self.qs, self.B)
        self.kernel(i)

    def step_is_kernel(self):
        return self.fold

    def config(self):
        return {"workload": "batched_decode", "requests": self.B, "tokens_per_step": self.B,
                "metadata": "folded into the fused launch" if self.fold else "separate launch",
                "history": "uniform[1,4096]", "H": 32, "D": 128, "ws": 32, "C": 1024,
                "W": 4, "block_size": 16, "activation": "silu", "residual": True,
                "graph": "hipGraph", "replicas": self.R}

    def oracle_sample(self, budget, threads=1):
        # Whole sub-batches of 256 requests, cycled, until the budget is spent.
        n_sub = self.R * self.B // 256

        def once(n):
            rows = slice(256 * (n % n_sub), 256 * (n % n_sub + 1))
            return 256, time_oracle_fused(sub_case(self.case, rows, rows), threads=threads)
        done, spent, n = repeat_until(budget, once)
        return (done / spent, f"{n} decode sub-batches of 256 requests ({done} tokens, cycling "
                f"the {n_sub} distinct ones)", spent)


class DecodeLayerBench(Workload):
    """Batched decode of all four conv streams of one layer (ws = 32 each,
    D = 128): one launch per step for the four streams, or one per stream."""

    STREAMS = [(0, 32), (32, 32), (64, 32), (96, 32)]

    def __init__(self, dev="cuda", requests: int = 256, one_launch: bool = True):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        self.one_launch = one_launch
        self.B = B = requests
        per_batch = 4 * B * 12_350
        self.R = max(2, -(-FLUSH_BYTES // per_batch) + 4 * (B <= 256))
        t = time.time()
        g = torch.Generator().manual_seed(6)
        ctx = [int(v) for v in torch.randint(1, 4097, (B * self.R,), generator=g)]
        self.cases = workloads.fused_streams_case(
            6, [1] * (B * self.R), ctx, H=32, D=128, streams=self.STREAMS, block_size=16, W=4,
            dtype="bf16", pool_blocks=int(B * self.R * 2 * 1.25) + 1, device=dev)
        c = self.cases[0]
        log(f"decode_layer: {self.R} batches of {B} requests x 4 streams in "
            f"{time.time() - t:.1f}s, cache {c.cache.numel() * c.cache.element_size() / 2**30:.1f} GiB")
        self.xs = [k.x.to(dev) for k in self.cases]
        self.ws_ = [k.weight.to(dev) for k in self.cases]
        self.cache = c.cache
        self.pos, self.sm, self.bt = c.positions.to(dev), c.slot_mapping.to(dev), c.block_table.to(dev)
        self.outs = [torch.empty_like(x) for x in self.xs]
        self.qsl = torch.arange(B + 1, dtype=torch.int32, device=dev)
        self.bytes_per_launch = (fused_streams_algorithmic_bytes(self.cases, (0, B))
                                 if one_launch else fused_algorithmic_bytes(c, (0, B)))
        self.tokens_per_step = B

    def rows(self, i):
        return slice(i * self.B, (i + 1) * self.B)

    def kernel(self, i):
        s, c = self.rows(i), self.cases[0]
        if self.one_launch:
            self.lib.sconv_fused_insert_conv_streams(
                [x[s] for x in self.xs], self.ws_, self.cache, self.pos[s], self.bt[s],
                self.sm[s], [o for o, _ in self.STREAMS], [w for _, w in self.STREAMS],
                c.block_size, "silu", True, query_start_loc=self.qsl, num_reqs=self.B,
                outs=[o[s] for o in self.outs])
            return
        for k, (off, ws) in enumerate(self.STREAMS):
            self.lib.sconv_fused_insert_conv_qsl(self.xs[k][s], self.ws_[k], self.cache,
                                                 self.pos[s], self.bt[s], self.qsl, self.B,
                                                 self.sm[s], off, ws, c.block_size, "silu", True,
                                                 out=self.outs[k][s])

    def kernels_per_call(self):
        return 1 if self.one_launch else 4

    def step(self, i):
        self.kernel(i)

    def step_is_kernel(self):
        return self.one_launch

    def config(self):
        return {"workload": "decode_layer", "requests": self.B, "tokens_per_step": self.B,
                "streams": 4, "stream_launches": "one launch for all 4 streams"
                if self.one_launch else "one launch per stream",
                "metadata": "folded into the fused launch", "history": "uniform[1,4096]",
                "H": 32, "D": 128, "ws": 32, "C_per_stream": 1024, "W": 4, "block_size": 16,
                "activation": "silu", "residual": True, "graph": "hipGraph", "replicas": self.R}

    def oracle_sample(self, budget, threads=1):
        # Whole sub-batches of 256 requests x 4 streams, cycled, until the
        # budget is spent.
        n_sub = self.R * self.B // 256

        def once(n):
            rows = slice(256 * (n % n_sub), 256 * (n % n_sub + 1))
            return 256, sum(time_oracle_fused(sub_case(k, rows, rows), threads=threads)
                            for k in self.cases)
        done, spent, n = repeat_until(budget, once)
        return (done / spent, f"{n} decode sub-batches of 256 requests x 4 streams ({done} tokens, "
                f"cycling the {n_sub} distinct ones)", spent)


class MixedPrefillBench(Workload):
    """Four streams of one layer convolved in turn over one shared cache."""

    def __init__(self, dev="cuda", fold: bool = False, one_launch: bool = False):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        self.fold = fold
        self.one_launch = one_launch
        t = time.time()
        self.streams = workloads.mixed_prefill_streams()
        b = self.streams[0]
        log(f"mixed_prefill: T={b.T} generated in {time.time() - t:.1f}s")
        self.bytes_per_launch = (fused_streams_algorithmic_bytes(self.streams) if one_launch
                                 else fused_algorithmic_bytes(b))
        self.R = 1   # one step moves ~4 x bytes_per_launch >> MALL
        self.cache = b.cache.to(dev)
        self.xs = [s.x.to(dev) for s in self.streams]
        self.ws_ = [s.weight.to(dev) for s in self.streams]
        self.outs = [torch.empty_like(x) for x in self.xs]
        self.pos, self.sm, self.bt = b.positions.to(dev), b.slot_mapping.to(dev), b.block_table.to(dev)
        self.qsl = b.query_start_loc.to(dev)
        self.si = torch.empty(b.T, dtype=torch.int32, device=dev)
        self.qs = torch.empty(b.T, dtype=torch.int32, device=dev)
        self.live = int((b.slot_mapping >= 0).sum())
        self.tokens_per_step = self.live

    def kernel(self, i):
        b = self.streams[0]
        if self.one_launch:
            meta = (dict(query_start_loc=self.qsl, num_reqs=b.num_reqs) if self.fold
                    else dict(seq_idx=self.si, query_start=self.qs))
            self.lib.sconv_fused_insert_conv_streams(
                self.xs, self.ws_, self.cache, self.pos, self.bt, self.sm,
                [st.off_s for st in self.streams], [st.ws for st in self.streams],
                b.block_size, "silu", True, outs=self.outs, **meta)
            return
        for s, st in enumerate(self.streams):
            if self.fold:
                self.lib.sconv_fused_insert_conv_qsl(self.xs[s], self.ws_[s], self.cache, self.pos,
                                                     self.bt, self.qsl, b.num_reqs, self.sm,
                                                     st.off_s, st.ws, b.block_size, "silu", True,
                                                     out=self.outs[s])
                continue
            self.lib.sconv_fused_insert_conv(self.xs[s], self.ws_[s], self.cache, self.pos, self.bt,
                                             self.si, self.sm, self.qs, st.off_s, st.ws,
                                             b.block_size, "silu", True, out=self.outs[s])

    def kernels_per_call(self):
        return 1 if self.one_launch else 4

    def step(self, i):
        b = self.streams[0]
        if not self.fold:
            self.lib.sconv_seq_metadata(self.qsl, b.num_reqs, b.num_actual, self.si, self.qs, b.T)
        self.kernel(i)

    def config(self):
        b = self.streams[0]
        return {"workload": "mixed_prefill", "requests": 16, "rows": b.T,
                "metadata": "folded into the fused launches" if self.fold else "separate launch",
                "stream_launches": "one launch for all 4 streams" if self.one_launch
                else "one launch per stream",
                "non_pad_tokens": self.live, "streams": 4, "H": 32, "D": 512, "ws": 128,
                "C": 4096, "W": 4, "block_size": 16, "pad_fraction": 0.1,
                "activation": "silu", "residual": True}

    def oracle_sample(self, budget, threads=1):
        # Whole streams (all rows), in turn, until the budget is spent; a
        # token counts once for its four streams.
        done, spent, n = repeat_until(
            budget, lambda n: (self.live / 4,
                               time_oracle_fused(self.streams[n % 4], threads=threads)))
        return done / spent, f"{n} whole-stream passes over all {self.live} live rows", spent


class SpecDecodeBench(Workload):
    """Speculative decode (512 x 4 drafts) plus the conv-window gather, in
    one launch (sconv_fused_insert_conv_gather) or in two."""

    B = 2048

    def __init__(self, dev="cuda", fold: bool = False, one_launch: bool = True):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        self.fold = fold
        self.one_launch = one_launch
        first = workloads.spec_decode()
        self.conv_bytes = fused_algorithmic_bytes(first)
        self.bytes_per_launch = self.conv_bytes
        self.R = max(2, -(-FLUSH_BYTES // self.bytes_per_launch) + 2)
        t = time.time()
        reqs = 512 * self.R
        self.case = workloads.spec_decode(device=dev, num_reqs=reqs,
                                          pool_blocks=int(reqs * 2 * 1.25) + 1)
        c = self.case
        log(f"spec_decode: {self.R} batches in {time.time() - t:.1f}s")
        self.x, self.w, self.cache = c.x.to(dev), c.weight.to(dev), c.cache
        self.pos, self.sm, self.bt = c.positions.to(dev), c.slot_mapping.to(dev), c.block_table.to(dev)
        self.out = torch.empty_like(self.x)
        self.qsl = torch.arange(0, self.B + 1, 4, dtype=torch.int32, device=dev)
        self.si = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.qs = torch.empty(self.B, dtype=torch.int32, device=dev)
        gc = workloads.spec_gather(first)
        self.gpos = gc.abs_positions.to(dev)
        # Each replica's gather reads its own live count, uniform in
        # [0, 512], from a fixed device buffer (as a replayed step would find
        # it rewritten on the device).
        g = torch.Generator().manual_seed(1004)
        self.counts = torch.randint(0, 513, (self.R,), generator=g).to(torch.int32)
        self.rcs = self.counts.to(dev)
        self.gout = torch.empty(self.R, 512, c.C, 3, dtype=torch.bfloat16, device=dev)
        self.tokens_per_step = self.B
        self.sweep = None
        if one_launch:
            # The launch also writes each live slot's window (2 x 4096
            # channels x 3 rows x 2 bytes) and reads its position; the
            # windows' source rows are x rows the conv reads anyway.
            self.bytes_per_launch = self.conv_bytes + int(
                round(float(self.counts.double().mean()) * (4096 * 3 * 2 + 4))) + 4

    def rows(self, i):
        return slice(i * self.B, (i + 1) * self.B)

    def kernel(self, i):
        s, c = self.rows(i), self.case
        bt = self.bt[512 * i:512 * (i + 1)]
        if self.one_launch:
            meta = (dict(query_start_loc=self.qsl, num_reqs=512) if self.fold
                    else dict(seq_idx=self.si, query_start=self.qs))
            x = self.x[s]
            self.lib.sconv_fused_insert_conv_gather(
                [x], [self.w], self.cache, self.pos[s], bt, self.sm[s], [c.off_s], [c.ws],
                c.block_size, x.view(1, self.B, -1), self.gpos, self.rcs[i:i + 1],
                self.gout[i], 3, activation="silu", use_residual=True, outs=[self.out[s]],
                **meta)
            return
        if self.fold:
            self.lib.sconv_fused_insert_conv_qsl(self.x[s], self.w, self.cache, self.pos[s], bt,
                                                 self.qsl, 512, self.sm[s], c.off_s, c.ws,
                                                 c.block_size, "silu", True, out=self.out[s])
            return
        self.lib.sconv_fused_insert_conv(self.x[s], self.w, self.cache, self.pos[s], bt, self.si,
                                         self.sm[s], self.qs, c.off_s, c.ws, c.block_size, "silu",
                                         True, out=self.out[s])

    def step(self, i):
        if not self.fold:
            self.lib.sconv_seq_metadata(self.qsl, 512, self.B, self.si, self.qs, self.B)
        self.kernel(i)
        if not self.one_launch:
            self.gather(i, self.rcs[i:i + 1])

    def step_is_kernel(self):
        return self.fold and self.one_launch

    def gather(self, i, count):
        self.lib.gather_intermediate_conv_window(self.x[self.rows(i)].view(1, self.B, -1),
                                                 self.gpos, count, self.gout[i], 3)

    def extra(self, stream, reps):
        """The window gather alone at fixed live counts (0, 128, 256, 512 of
        512 slots), us per launch from HIP events around graph replays: what
        a dead slot costs next to a live one."""
        import torch
        out = {}
        for n in (0, 128, 256, 512):
            rc = torch.tensor([n], dtype=torch.int32, device="cuda")
            g = capture(lambda i: self.gather(i, rc), range(self.R), stream)
            upload(g, stream)
            time_graph(g, 1, stream)
            us = time_graph(g, reps, stream) * 1e3 / (reps * self.R)
            out[str(n)] = {"us": round(us, 3),
                           # 2 x 4096 channels x 3 rows x 2 bytes + 4 per live slot
                           "GB/s": round(49156 * n / (us * 1e-6) / 1e9, 1) if n else None}
        self.sweep = out
        return {"gather_real_count_sweep": out}

    def config(self):
        return {"workload": "spec_decode", "requests": 512, "drafts": 4, "tokens_per_step": 2048,
                "metadata": "folded into the fused launch" if self.fold else "separate launch",
                "gather_launch": "in the conv's launch (sconv_fused_insert_conv_gather)"
                if self.one_launch else "its own launch after the conv's",
                "positions": "uniform[1,131072)", "H": 64, "D": 64, "ws": 64, "C": 4096,
                "W": 4, "block_size": 32,
                "gather": {"max_count": 512, "d_conv": 3,
                           "real_count": "uniform[0,512] per replica, on the device",
                           "mean_real_count": round(float(self.counts.float().mean()), 1)},
                "activation": "silu", "residual": True, "graph": "hipGraph",
                "replicas": self.R}

    def oracle_sample(self, budget, threads=1):
        def once(n):
            i = n % self.R
            sub = sub_case(self.case, self.rows(i), slice(512 * i, 512 * (i + 1)))
            return self.B, time_oracle_fused(sub, threads=threads)
        done, spent, n = repeat_until(budget, once)
        return (done / spent, f"fused conv of {n} whole spec batches ({done} tokens, cycling the "
                f"{self.R} distinct ones)", spent)


class SsmPrefillBench(Workload):
    kernel_name = "varlen_fwd_kernel"

    def __init__(self, dev="cuda"):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        t = time.time()
        self.case = workloads.ssm_varlen()
        c = self.case
        log(f"ssm_prefill generated in {time.time() - t:.1f}s")
        self.R = 1   # one step moves ~1.07 GB
        self.x = c.x.to(dev)
        self.out = torch.empty_like(self.x)
        self.w, self.b = c.weight.to(dev), c.bias.to(dev)
        self.st = c.conv_states.to(dev)
        self.qsl = c.query_start_loc.to(dev)
        self.ci = c.cache_indices.to(dev)
        self.hi = c.has_initial_state.to(dev)
        dim, T = c.x.shape
        e = 2
        n_init = int(c.has_initial_state.sum())
        self.bytes_per_launch = (2 * dim * T + (n_init + 8) * dim * 3 + dim * 5) * e + 4 * 9
        self.tokens_per_step = T

    def kernel(self, i):
        self.lib.causal_conv1d_varlen_fwd(self.x, self.w, self.b, self.st, self.qsl, self.ci,
                                          self.hi, True, -1, out=self.out)

    step = kernel

    def config(self):
        return {"workload": "ssm_prefill", "sequences": 8, "seq_len": 4096, "dim": 8192,
                "W": 4, "layout": "channel-major", "state_slots": 1024, "with_state": 4,
                "activation": "silu", "bias": True}

    def oracle_sample(self, budget, threads=1):
        import oracle
        from tests.helpers import to_np
        c = self.case
        import numpy as np
        # Pairs of sequences (one with a state, one without), in turn, all
        # channels, until the budget is spent.
        with_st = [int(v) for v in torch_where(c.has_initial_state)]
        without = [int(v) for v in torch_where(~c.has_initial_state)]
        L = 4096
        xs = to_np(c.x)
        w, b, st, ci, hi = (to_np(c.weight), to_np(c.bias), to_np(c.conv_states),
                            to_np(c.cache_indices), to_np(c.has_initial_state))

        def once(n):
            keep = [with_st[n % len(with_st)], without[n % len(without)]]
            x2 = np.ascontiguousarray(np.concatenate([xs[:, k * L:(k + 1) * L] for k in keep], 1))
            t0 = time.perf_counter()
            oracle.causal_conv1d_varlen_fwd(x2, w, b, st, np.array([0, L, 2 * L], np.int32),
                                            ci[keep], hi[keep], "silu", -1, threads=threads)
            return 2 * L, time.perf_counter() - t0
        done, spent, n = repeat_until(budget, once)
        return (done / spent, f"{n} pairs of 4096-token sequences, one with a state and one "
                f"without ({done} tokens, all channels)", spent)


class SsmDecodeBench(Workload):
    kernel_name = "update_kernel"
    oracle_split = False

    def __init__(self, dev="cuda"):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        c = workloads.ssm_varlen()
        self.case = c
        xs = workloads.update_inputs(3, 64, 8, 8192)
        self.R = 64
        self.x = torch.stack(xs).to(dev)
        self.out = torch.empty_like(self.x)
        self.w, self.b = c.weight.to(dev), c.bias.to(dev)
        self.st = c.conv_states.to(dev)
        self.ci = c.cache_indices.to(dev)
        self.bytes_per_launch = (8 * 8192 * 2 + 8 * 8192 * 3 * 2) * 2 + 8192 * 5 * 2 + 32
        self.tokens_per_step = 8

    def kernel(self, i):
        self.lib.causal_conv1d_update(self.x[i], self.st, self.w, self.b, True, None, self.ci, -1,
                                      out=self.out[i])

    step = kernel

    def config(self):
        return {"workload": "ssm_decode", "batch": 8, "dim": 8192, "W": 4,
                "state_slots": 1024, "activation": "silu", "bias": True,
                "graph": "hipGraph", "steps_per_graph": 64}

    def oracle_sample(self, budget, threads=1):
        import oracle
        from tests.helpers import to_np
        c = self.case
        st, w, b, ci = (to_np(c.conv_states), to_np(c.weight), to_np(c.bias),
                        to_np(c.cache_indices))
        xs = [to_np(self.x[i]) for i in range(min(self.R, 8))]

        def once(n):
            t0 = time.perf_counter()
            oracle.causal_conv1d_update(xs[n % len(xs)], st, w, b, "silu", ci, -1)
            return 8, time.perf_counter() - t0
        done, spent, n = repeat_until(budget, once)
        return done / spent, f"{n} decode steps of 8 rows ({done} tokens)", spent


class SsmSpecDecodeBench(Workload):
    """Speculative decode on the SSM state pool: 8 rows x 4 draft tokens of
    dim 8192 per step against ring states (W-1 columns, positions
    uniform[0, 4096)), through causal_conv1d_update_tokens; 64 steps per
    graph, each with its own inputs and outputs."""
    kernel_name = "update_tokens_vec_kernel"
    oracle_split = False
    B, T, DIM, W, STEPS = 8, 4, 8192, 4, 64

    def __init__(self, dev="cuda"):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        c = workloads.ssm_varlen()
        self.case = c
        g = torch.Generator().manual_seed(11)
        self.R = self.STEPS
        # x [R, batch, T, dim] with channels contiguous, viewed [batch, dim, T]
        self.x = torch.randn(self.R, self.B, self.T, self.DIM, generator=g).to(torch.bfloat16).to(dev)
        self.out = torch.empty_like(self.x)
        self.w, self.b = c.weight.to(dev), c.bias.to(dev)
        self.st = c.conv_states.to(dev)
        self.ci = c.cache_indices.to(dev)
        self.seqlens = torch.randint(0, 4096, (self.R, self.B), generator=g).to(torch.int32).to(dev)
        e = 2
        self.bytes_per_launch = (2 * self.B * self.T * self.DIM * e        # x in, out
                                 + 2 * self.B * self.DIM * (self.W - 1) * e  # state in, out
                                 + self.DIM * (self.W + 1) * e + 8 * self.B)
        self.tokens_per_step = self.B * self.T

    def kernel(self, i):
        self.lib.causal_conv1d_update_tokens(self.x[i].permute(0, 2, 1), self.st, self.w, self.b,
                                             True, self.seqlens[i], self.ci, -1,
                                             out=self.out[i].permute(0, 2, 1))

    step = kernel

    def config(self):
        return {"workload": "ssm_spec_decode", "batch": self.B, "draft_tokens": self.T,
                "dim": self.DIM, "W": self.W, "state": "ring, W-1 columns",
                "positions": "uniform[0,4096)", "state_slots": 1024, "activation": "silu",
                "bias": True, "graph": "hipGraph", "steps_per_graph": self.STEPS}

    def oracle_sample(self, budget, threads=1):
        import oracle
        from tests.helpers import to_np
        c = self.case
        st, w, b, ci = (to_np(c.conv_states), to_np(c.weight), to_np(c.bias),
                        to_np(c.cache_indices))
        steps = [(to_np(self.x[i].permute(0, 2, 1).cpu()), to_np(self.seqlens[i].cpu()))
                 for i in range(min(self.R, 8))]

        def once(n):
            x, sl = steps[n % len(steps)]
            t0 = time.perf_counter()
            oracle.causal_conv1d_update_tokens(x, st, w, b, "silu", sl, ci, -1)
            return self.B * self.T, time.perf_counter() - t0
        done, spent, n = repeat_until(budget, once)
        return done / spent, f"{n} steps of 8 rows x 4 tokens ({done} tokens)", spent


class SsmStateGatherBench(Workload):
    """Prefix-cache extraction of SSM states: 96 live of 128 slots, each a
    whole state row (64 heads x 64 x 128 fp32 = 2 MiB) gathered from 128
    chunk states at distinct indices; three replicas, so a step reads HBM,
    not the MALL."""
    unit = "slots/s"
    kernel_name = "gather_ssm_kernel"
    dtype = "f32"
    oracle_split = False
    SHAPE = (64, 64, 128)
    CHUNKS, SLOTS, LIVE, R_ = 128, 128, 96, 3

    def __init__(self, dev="cuda"):
        import torch

        import depthwise_causal_conv1d_amd as lib
        self.lib = lib
        g = torch.Generator().manual_seed(8)
        self.R = self.R_
        self.states = [torch.randn((self.CHUNKS,) + self.SHAPE, generator=g).to(dev)
                       for _ in range(self.R)]
        # Distinct source rows: a repeated row would be served from cache.
        self.idx = [torch.randperm(self.CHUNKS, generator=g)[:self.SLOTS].to(dev)
                    for _ in range(self.R)]
        self.out = [torch.empty((self.SLOTS,) + self.SHAPE, device=dev) for _ in range(self.R)]
        self.rc = torch.tensor([self.LIVE], dtype=torch.int32, device=dev)
        row = 4 * self.SHAPE[0] * self.SHAPE[1] * self.SHAPE[2]
        self.bytes_per_launch = 2 * self.LIVE * row + 8 * self.LIVE + 4
        self.tokens_per_step = self.LIVE  # one unit per extracted slot

    def kernel(self, i):
        self.lib.gather_intermediate_ssm_state(self.states[i], self.idx[i], self.rc, self.out[i])

    step = kernel

    def config(self):
        return {"workload": "ssm_state_gather", "unit_per_token": "one extracted slot",
                "num_chunks": self.CHUNKS, "max_count": self.SLOTS, "real_count": self.LIVE,
                "state_shape": list(self.SHAPE), "state_dtype": "f32", "graph": "hipGraph",
                "replicas": self.R}

    def oracle_sample(self, budget, threads=1):
        import oracle
        st = self.states[0][:16].cpu().numpy()
        idx = (self.idx[0].cpu() % 16).numpy()
        out0 = self.out[0][:32].cpu().numpy()

        def once(n):
            t0 = time.perf_counter()
            oracle.gather_ssm_state(st, idx, 32, out0)
            return 32, time.perf_counter() - t0
        done, spent, n = repeat_until(budget, once)
        return done / spent, f"{n} gathers of 32 slots from 16 chunk states ({done} slots)", spent


def torch_where(mask):
    import torch
    return torch.nonzero(mask).flatten()


WORKLOADS = {
    "batched_decode": DecodeBench,
    "decode_layer": DecodeLayerBench,
    "mixed_prefill": MixedPrefillBench,
    "spec_decode": SpecDecodeBench,
    "ssm_prefill": SsmPrefillBench,
    "ssm_decode": SsmDecodeBench,
    "ssm_spec_decode": SsmSpecDecodeBench,
    "ssm_state_gather": SsmStateGatherBench,
}

DEFAULT_STEPS = {"batched_decode": 19200, "decode_layer": 9600, "mixed_prefill": 200,
                 "spec_decode": 2000, "ssm_prefill": 200, "ssm_decode": 6400,
                 "ssm_spec_decode": 6400, "ssm_state_gather": 600}


# ---------------------------------------------------------------- timing

def capture(fn, indices, stream):
    """One hipGraph of fn(i) for i in indices, captured on `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in indices:
                fn(i)
    return g


_HIP = None


def hip_runtime():
    """The HIP runtime torch loaded (one per process)."""
    global _HIP
    if _HIP is None:
        import ctypes
        _HIP = ctypes.CDLL("libamdhip64.so.7")
        _HIP.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return _HIP


def upload(graph, stream):
    """Upload an instantiated graph to the device without running it, so
    that its first replay does no set-up work."""
    rc = hip_runtime().hipGraphUpload(graph.raw_cuda_graph_exec(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"hipGraphUpload failed ({rc})")


def time_graph(graph, reps, stream):
    """Milliseconds of `reps` back-to-back replays of an uploaded graph,
    between HIP events on `stream`; a spin kernel queued first keeps the
    host's submission out of the interval."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


SPIN_CYCLES = 2_000_000   # ~1 ms of spinning ahead of a timed interval
OTHER_LIB = None          # path of a library other than the in-tree build (--lib)
PROFILED_FORM = True      # the run uses the launch forms the committed profiles were taken on


class StepGraphs:
    """The graphs of one workload: K timed steps, W warm-up steps (replicas
    cycled), and R launches of the dominant kernel alone."""

    def __init__(self, wl, K, Wm, stream):
        self.wl, self.K, self.Wm, self.stream = wl, K, Wm, stream
        R = wl.R
        self.full = capture(wl.step, range(R), stream) if max(K, Wm) >= R else None
        self.k_rem = capture(wl.step, range(K % R), stream) if K % R else None
        # Warm-up steps end on replica R-1, so the timed steps, which start
        # on replica 0, find none of their bytes left in a cache.
        self.w_rem = (capture(wl.step, range(R - Wm % R, R), stream) if Wm % R else None)
        self.kern = capture(wl.kernel, range(R), stream)
        for g in (self.full, self.k_rem, self.w_rem, self.kern):
            if g is not None:
                upload(g, stream)

    def _run(self, n, rem):
        for _ in range(n // self.wl.R):
            self.full.replay()
        if rem is not None:
            rem.replay()

    def warmup(self):
        import torch
        with torch.cuda.stream(self.stream):
            self._run(self.Wm, self.w_rem)
        torch.cuda.synchronize()

    def timed(self):
        """(event ms, wall s) of exactly K steps."""
        import torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.stream):
            torch.cuda._sleep(SPIN_CYCLES)
            e0.record(self.stream)
            self._run(self.K, self.k_rem)
            e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1), wall

    def kernel_us(self, reps):
        """Average duration of one launch of the dominant kernel (us), after
        one untimed replay of its graph."""
        time_graph(self.kern, 1, self.stream)
        ms = time_graph(self.kern, reps, self.stream)
        return ms * 1e3 / (reps * self.wl.R * self.wl.kernels_per_call())


def cpu_baseline(wl, budget):
    """The oracle on every host core the process may use, and alone."""
    if budget <= 0:
        return None
    n = cpu_threads() if wl.oracle_split else 1
    v, sample, spent = wl.oracle_sample(budget, threads=n)
    # the GPU step's algorithmic bytes per unit, applied to the oracle's rate
    per_unit = wl.bytes_per_launch * wl.kernels_per_call() / wl.tokens_per_step
    out = {"value": round(v, 1), "unit": wl.unit, "cores": n, "kind": "oracle",
           "GBs": round(v * per_unit / 1e9, 3),
           "sample": f"{sample}; {spent:.1f} s on {n} thread{'s' if n > 1 else ''}",
           "hardware_concurrency": os.cpu_count(), "cpu_model": cpu_model()}
    if n > 1:
        v1, sample1, spent1 = wl.oracle_sample(budget, threads=1)
        out["single_thread"] = {"value": round(v1, 1), "cores": 1,
                                "GBs": round(v1 * per_unit / 1e9, 3),
                                "sample": f"{sample1}; {spent1:.1f} s on 1 thread"}
    return out


def measure(wl, name, K, Wm, reps, budget, stream):
    """Everything one JSON line says about one workload."""
    graphs = StepGraphs(wl, K, Wm, stream)
    graphs.warmup()
    ms, wall = graphs.timed()
    kern_us = graphs.kernel_us(reps)
    extra = wl.extra(stream, reps) if hasattr(wl, "extra") else {}
    achieved = wl.bytes_per_launch / (kern_us * 1e-6) / 1e9
    # Stored trace and counter figures describe the in-tree build, in the
    # default launch forms and batch size, only.
    stored = PROFILED_FORM and not OTHER_LIB
    trace_us = stored_trace(wl.kernel_name, name) if stored else None
    roof = {"bound": wl.bound, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_trace": (round(wl.bytes_per_launch / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                           if trace_us else None),
            "headline": "frac: HIP events around graph replays of the kernel alone",
            "traffic": stored_traffic(name, wl.kernel_name) if stored else None,
            "kernel": wl.kernel_name,
            "bytes_per_launch": wl.bytes_per_launch, "launch_us": round(kern_us, 3),
            "launch_us_trace": trace_us,
            # the same bytes over the event-timed step, where a step is one
            # launch of the kernel and nothing else
            "step_frac": round(wl.bytes_per_launch / (ms * 1e-3 / K) / 1e9 / HBM_PEAK_GBS, 4)
            if wl.step_is_kernel() else None}
    line = {
        "value": round(wl.tokens_per_step * K / (ms * 1e-3), 1),
        "unit": wl.unit,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms / K, 6),
        "wall_ms_per_step": round(wall * 1e3 / K, 6),
        "dtype": wl.dtype,
        "config": wl.config(),
        "roofline": roof,
        "cpu_baseline": cpu_baseline(wl, budget),
    }
    line.update(extra)
    return line


# ---------------------------------------------------------------- probes

PROBE_SRC = os.path.join(ROOT, "bench_probes.hip")
PROBE_LIB = os.path.join(ROOT, "bench_probes.so")
PROBE_LIB_PRELOAD = os.path.join(ROOT, "bench_probes_preload.so")


def build_probes(verbose=False) -> str:
    """Compile the measurement probes (bench_probes.hip) for gfx950, twice:
    as they are, and with their leading kernel arguments preloaded into
    SGPRs by the compiler (PROBE_LIB_PRELOAD), so that the latency floors
    show what an argument load costs at the decode launch shape."""
    import subprocess

    from depthwise_causal_conv1d_amd import build as b
    for out, extra in ((PROBE_LIB, []),
                       (PROBE_LIB_PRELOAD, ["-mllvm", "-amdgpu-kernarg-preload-count=16"])):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [b.hipcc(), f"--offload-arch={b.ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *extra,
               "-o", tmp, PROBE_SRC]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
        os.replace(tmp, out)
    return PROBE_LIB


def _probe_lib(path=None):
    import ctypes
    path = path or PROBE_LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import bench; "
                          "bench.build_probes()'` (or __graft_entry__.build())")
    P = ctypes.CDLL(path)
    V, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    U32 = ctypes.c_uint32
    P.probe_read.argtypes = [V, I64, V, I64, I32, U32, V]
    P.probe_write.argtypes = [V, I64, I64, I32, I32, U32, V]
    P.probe_copy.argtypes = [V, V, I64, I64, I32, I32, U32, V]
    P.probe_read_write2.argtypes = [V, V, V, I64, I32, I32, I64, I32, I32, U32, V]
    P.probe_prefill_layout.argtypes = [V, V, V, V, I32, I32, I32, U32, V]
    P.probe_empty.argtypes = [I32, V]
    P.probe_load_store.argtypes = [V, V, I32, V]
    P.probe_chain.argtypes = [V, I32, V, V, V, I32, I32, V]
    return P


def _ok(rc):
    if rc != 0:
        raise RuntimeError(f"probe launch failed ({rc})")


# Shapes of the streaming probes: (vectors of 16 bytes per lane and pass,
# vectors per 256-thread workgroup).  Which one is fastest depends on the
# pattern and the size, so each ceiling is the best of them, with streaming
# and with ordinary stores, at full occupancy and at 5 and 4 workgroups per
# CU (dynamic LDS the kernels do not use: 160 KiB per CU).
PROBE_SHAPES = ((1, 256), (2, 512), (4, 1024), (2, 2048))
PROBE_LDS = (0, 32768, 40960)
LDS_PER_CU = 163840


def _occupancy(lds):
    return "full" if lds == 0 else f"{LDS_PER_CU // lds} workgroups per CU"


def _time_launches(fn, R, stream):
    """Milliseconds per launch of fn(0..R-1), captured as one graph and
    replayed back to back (after two untimed replays)."""
    g = capture(fn, range(R), stream)
    upload(g, stream)
    time_graph(g, 2, stream)
    reps = max(5, 40 // R)
    ms = time_graph(g, reps, stream) / (reps * R)
    del g
    return ms


def prefill_layout(P, stream, T=18432):
    """TB/s of the mixed prefill's own traffic in its own layout (one stream
    launch of T rows, C = 4096 bf16, sequential slots; bench_probes.hip),
    alone and with the conv's other loads (3 halo rows, 4 filter-tap
    vectors per lane), each the best of the PROBE_LDS occupancies.  Bytes
    are the algorithmic ones: x read, out written, cache pieces written."""
    import torch
    R = 2
    xb, cb = T * 512 * 16, T * 2048 * 16
    x = torch.empty(R * xb, dtype=torch.uint8, device="cuda").fill_(1)
    o = torch.empty(R * xb, dtype=torch.uint8, device="cuda")
    c = torch.empty(R * cb, dtype=torch.uint8, device="cuda")
    w = torch.empty(2048 * 16, dtype=torch.uint8, device="cuda").fill_(2)
    s = stream.cuda_stream
    res = {}
    for halo, wts in ((0, 0), (0, 4), (3, 0), (3, 4)):
        runs = []
        for lds in PROBE_LDS:
            ms = _time_launches(lambda i: _ok(P.probe_prefill_layout(
                x.data_ptr() + i * xb, w.data_ptr(), o.data_ptr() + i * xb,
                c.data_ptr() + i * cb, T, halo, wts, lds, s)), R, stream)
            runs.append((round(3 * xb / (ms * 1e-3) / 1e12, 3), _occupancy(lds), round(ms * 1e3, 2)))
        tbs, occ, us = max(runs)
        name = {(0, 0): "traffic", (0, 4): "traffic_and_taps", (3, 0): "traffic_and_halo",
                (3, 4): "traffic_taps_and_halo"}[(halo, wts)]
        res[name] = {"TB/s": tbs, "us": us, "occupancy": occ}
    res["rows"] = T
    res["bytes"] = 3 * xb
    del x, o, c, w
    torch.cuda.empty_cache()
    return res


def stream_ceilings(P, stream, names, n16=None, forms=False):
    """TB/s of the streaming reference kernels `names`, each the best of
    PROBE_SHAPES x {streaming, ordinary stores} x PROBE_LDS, timed with HIP
    events over graph replays.  Each stream moves n16 vectors of 16 bytes (default
    1 GiB); smaller streams cycle through replicas at least 1 GiB apart, so
    that every launch reads HBM.  forms: also list every form's figure."""
    import torch
    GiB = 1 << 30
    n16 = GiB // 16 if n16 is None else int(n16)
    if n16 < 16 or n16 % 16 or 16 * n16 > GiB:
        raise ValueError(f"stream of {n16} vectors: need a multiple of 16 up to 1 GiB")
    R = GiB // (16 * n16)
    s = stream.cuda_stream
    a = torch.empty(GiB, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(GiB, dtype=torch.uint8, device="cuda")
    c = torch.empty(GiB, dtype=torch.uint8, device="cuda")
    d = torch.empty(4 * GiB, dtype=torch.uint8, device="cuda")  # 256-byte pieces of 1 KiB rows
    sink = torch.empty(256 * 16, dtype=torch.uint8, device="cuda")
    nb = 16 * n16

    def case(name, i, per, u, nt, lds):
        A, B, C, Dd = (x.data_ptr() + i * k * nb for x, k in ((a, 1), (b, 1), (c, 1), (d, 4)))
        if name == "read":
            return P.probe_read(A, n16, sink.data_ptr(), per, u, lds, s)
        if name == "write":
            return P.probe_write(B, n16, per, u, nt, lds, s)
        if name == "copy":
            return P.probe_copy(A, B, n16, per, u, nt, lds, s)
        if name == "read_write2_linear":
            return P.probe_read_write2(A, B, C, n16, 1024, 1024, per, u, nt, lds, s)
        return P.probe_read_write2(A, B, Dd, n16, 256, 1024, per, u, nt, lds, s)

    moved = {"read": 1, "write": 1, "copy": 2, "read_write2_linear": 3,
             "read_write2_pieces_256_of_1024": 3}
    res = {}
    for name in names:
        runs = []
        for u, per in PROBE_SHAPES:
            for nt in ((1,) if name == "read" else (1, 0)):
                for lds in PROBE_LDS:
                    ms = _time_launches(lambda i: _ok(case(name, i, per, u, nt, lds)), R, stream)
                    nbytes = moved[name] * nb
                    runs.append({"lane_vectors": u, "workgroup_KiB": per * 16 // 1024,
                                 "stores": "streaming" if nt else "ordinary",
                                 "occupancy": _occupancy(lds),
                                 "TB/s": round(nbytes / (ms * 1e-3) / 1e12, 3),
                                 "ms": round(ms, 4)})
        best = max(runs, key=lambda r: r["TB/s"])
        res[name] = {"TB/s": best["TB/s"],
                     "frac_of_peak": round(best["TB/s"] * 1e3 / HBM_PEAK_GBS, 4),
                     "ms": best["ms"], "bytes": moved[name] * nb,
                     "form": {k: best[k] for k in ("lane_vectors", "workgroup_KiB", "stores",
                                                   "occupancy")}}
        if forms:
            res[name]["forms"] = runs
    del a, b, c, d, sink
    torch.cuda.empty_cache()
    return res


def decode_floors(P, stream, names):
    """µs per launch of the latency probes `names` at the decode launch
    shape: 512 waves, one per workgroup; 512 launches per graph, each on its
    own 512 KiB of input and output."""
    import torch
    waves, R, s = 512, 512, stream.cuda_stream
    src = torch.empty(R * waves * 64 * 16, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    g = torch.Generator().manual_seed(5)
    # table rows name blocks of `data` in entry 0; entries 64, 128, 192 are 0
    table = torch.randint(0, 16384, (R * waves, 256), generator=g).to(torch.int32)
    table[:, 64] = 0
    table[:, 128] = 0
    table[:, 192] = 0
    table = table.to("cuda")
    meta = torch.arange(R * waves, dtype=torch.int32, device="cuda")
    data = torch.empty(16384 * 8192 * 16, dtype=torch.uint8, device="cuda").fill_(4)
    probes = {
        "empty": lambda i: _ok(P.probe_empty(waves, s)),
        "load_store": lambda i: _ok(P.probe_load_store(src.data_ptr() + i * waves * 1024,
                                                       dst.data_ptr() + i * waves * 1024,
                                                       waves, s)),
        "table_row": lambda i: _ok(P.probe_chain(
            None, i * waves, table.data_ptr(), data.data_ptr(),
            dst.data_ptr() + i * waves * 1024, waves, 0, s)),
        "table_row_then_3_tap_rows": lambda i: _ok(P.probe_chain(
            None, i * waves, table.data_ptr(), data.data_ptr(),
            dst.data_ptr() + i * waves * 1024, waves, 3, s)),
        "meta_then_table_row": lambda i: _ok(P.probe_chain(
            meta.data_ptr() + i * waves * 4, 0, table.data_ptr(), data.data_ptr(),
            dst.data_ptr() + i * waves * 1024, waves, 0, s)),
        "meta_table_row_then_3_tap_rows": lambda i: _ok(P.probe_chain(
            meta.data_ptr() + i * waves * 4, 0, table.data_ptr(), data.data_ptr(),
            dst.data_ptr() + i * waves * 1024, waves, 3, s)),
    }
    lat = {}
    for name in names:
        gr = capture(probes[name], range(R), stream)
        upload(gr, stream)
        time_graph(gr, 1, stream)
        lat[name] = round(time_graph(gr, 3, stream) * 1e3 / (3 * R), 3)
    del src, dst, table, meta, data
    torch.cuda.empty_cache()
    return lat


# One mixed-prefill stream launch (16 requests, 4 streams of C = 4096) moves
# 469.7 MB: the prefill pattern is also measured at that size, as read n :
# write 2n.
PREFILL_LAUNCH_BYTES = 469_712_208


def _launch_n16(launch_bytes):
    return int(launch_bytes) // 3 // 256 * 16


def run_probes(stream):
    """Streaming ceilings and latency floors of this GPU (one JSON line)."""
    P = _probe_lib()
    res = {"workload": "probe", "peak_GBs": HBM_PEAK_GBS,
           "shapes": [{"lane_vectors": u, "workgroup_KiB": per * 16 // 1024}
                      for u, per in PROBE_SHAPES]}
    res.update(stream_ceilings(P, stream, ["read", "write", "copy", "read_write2_linear",
                                           "read_write2_pieces_256_of_1024"], forms=True))
    at = stream_ceilings(P, stream, ["read_write2_pieces_256_of_1024"],
                         n16=_launch_n16(PREFILL_LAUNCH_BYTES), forms=True)
    res["read_write2_pieces_256_of_1024_at_prefill_launch_size"] = at[
        "read_write2_pieces_256_of_1024"]
    res["prefill_layout"] = prefill_layout(P, stream)
    floors = ["empty", "load_store", "table_row", "table_row_then_3_tap_rows",
              "meta_then_table_row", "meta_table_row_then_3_tap_rows"]
    res["decode_shape_floors_us"] = decode_floors(P, stream, floors)
    # the same probes with their kernel arguments preloaded into SGPRs
    res["decode_shape_floors_us_args_preloaded"] = decode_floors(
        _probe_lib(PROBE_LIB_PRELOAD), stream, floors)
    res["decode_shape"] = {"waves": 512, "threads_per_workgroup": 64, "launches_per_graph": 512}
    return res


def machine_reference(stream, prefill_launch_bytes=PREFILL_LAUNCH_BYTES):
    """What the same GPU reaches on the headline's patterns, for the default
    line: the copy and the mixed prefill's write patterns (TB/s; the pieces
    pattern at 1 GiB per stream and at the prefill launch's own size), and
    the decode kernel's dependent chain at its launch shape (µs), with its
    kernel arguments preloaded into SGPRs as the fused kernel's are.  None
    when the probe kernels are not built."""
    try:
        P = _probe_lib()
    except ImportError as e:
        log(f"machine reference skipped: {e}")
        return None
    c = stream_ceilings(P, stream, ["copy", "read_write2_linear",
                                    "read_write2_pieces_256_of_1024"])
    at = stream_ceilings(P, stream, ["read_write2_pieces_256_of_1024"],
                         n16=_launch_n16(prefill_launch_bytes))["read_write2_pieces_256_of_1024"]
    lay = prefill_layout(P, stream)
    f = decode_floors(P, stream, ["empty", "table_row_then_3_tap_rows"])
    # The fused kernel takes its first-hop values as leading arguments that
    # the hardware preloads into SGPRs: its floor is the chain probe built
    # the same way (the unpreloaded chain is reported beside it).
    try:
        fp = decode_floors(_probe_lib(PROBE_LIB_PRELOAD), stream, ["table_row_then_3_tap_rows"])
    except ImportError as e:  # the preloaded build of the probes is missing
        log(f"preloaded decode floor skipped: {e}")
        fp = f
    pieces = c["read_write2_pieces_256_of_1024"]
    return {"source": "bench_probes.hip in this run (bench.py --probe measures all)",
            "forms": "best of %d workgroup shapes x 2 store forms x %d occupancies" % (
                len(PROBE_SHAPES), len(PROBE_LDS)),
            "copy_TBs": c["copy"]["TB/s"],
            "prefill_pattern_linear_TBs": c["read_write2_linear"]["TB/s"],
            "prefill_pattern_TBs": pieces["TB/s"],
            "prefill_pattern_form": pieces["form"],
            "prefill_pattern_at_launch_size_TBs": at["TB/s"],
            "prefill_pattern_at_launch_size_form": at["form"],
            "prefill_layout_TBs": lay["traffic"]["TB/s"],
            "prefill_layout_with_taps_and_halo_TBs": lay["traffic_taps_and_halo"]["TB/s"],
            "empty_launch_us": f["empty"],
            "decode_chain_floor_us": fp["table_row_then_3_tap_rows"],
            "decode_chain_floor_us_args_loaded": f["table_row_then_3_tap_rows"]}


# ---------------------------------------------------------------- main

def make_workload(name, args):
    fold = (args.metadata == "folded" or
            (args.metadata == "auto" and name in ("batched_decode", "spec_decode")))
    one = (args.stream_launches == "one" or
           (args.stream_launches == "auto" and name == "decode_layer"))
    if name == "batched_decode":
        return DecodeBench(requests=args.requests, fold=fold)
    if name == "decode_layer":
        return DecodeLayerBench(requests=args.requests, one_launch=one)
    if name == "mixed_prefill":
        return MixedPrefillBench(fold=fold, one_launch=one)
    if name == "spec_decode":
        return SpecDecodeBench(fold=fold, one_launch=args.gather_launch != "separate")
    return WORKLOADS[name]()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="default", choices=["default"] + sorted(WORKLOADS),
                    help="default: batched decode, with the mixed prefill in a `prefill` "
                         "object of the same line")
    ap.add_argument("--probe", action="store_true",
                    help="measure this GPU's streaming ceilings and decode-shape latency "
                         "floors instead (one JSON line)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time per CPU-baseline leg (0: skip)")
    ap.add_argument("--metadata", choices=("auto", "separate", "folded"), default="auto",
                    help="per-row request search: its own sconv_seq_metadata launch per step, "
                         "or inside the fused launch (sconv_fused_insert_conv_qsl); auto picks "
                         "the faster per step: folded for decode and spec decode, separate for "
                         "the 4-stream prefill (one metadata launch serves four streams)")
    ap.add_argument("--requests", type=int, default=256,
                    help="batched_decode and decode_layer: requests per decode batch")
    ap.add_argument("--stream-launches", choices=("auto", "one", "separate"), default="auto",
                    help="decode_layer and mixed_prefill: all four streams of the layer in one "
                         "sconv_fused_insert_conv_streams launch, or one launch per stream; "
                         "auto: one for decode_layer, separate (the configured four calls) "
                         "for mixed_prefill")
    ap.add_argument("--gather-launch", choices=("same", "separate"), default="same",
                    help="spec_decode: the window gather in the conv's launch "
                         "(sconv_fused_insert_conv_gather) or in its own launch after it")
    ap.add_argument("--lib", default=None,
                    help="measure another build of libsconv.so (one made with "
                         "`python -m depthwise_causal_conv1d_amd.build --define ... --out PATH`)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()
    if args.steps is not None and args.steps < 1:
        ap.error("--steps must be at least 1")
    if args.warmup is not None and args.warmup < 0:
        ap.error("--warmup must be non-negative")
    if args.requests < 1:
        ap.error("--requests must be at least 1")
    if args.gpus != 1:
        print("bench.py measures one GPU only: libsconv has no multi-GPU path "
              "(the op shards per request or per head with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    if args.probe:
        print(json.dumps(run_probes(stream)), flush=True)
        return
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        evict = torch.empty(4 * n, dtype=torch.uint8, device="cuda").fill_(2)  # push src out of L2/MALL
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read, {n} bytes written")
        del src, dst, evict

    import depthwise_causal_conv1d_amd as lib
    global PROFILED_FORM
    PROFILED_FORM = (args.metadata == "auto" and args.stream_launches == "auto" and
                     args.gather_launch == "same" and args.requests == 256)
    if args.lib:
        global OTHER_LIB
        from depthwise_causal_conv1d_amd import _lib
        OTHER_LIB = _lib.LIB_PATH = os.path.abspath(args.lib)
    lib.sconv_init()
    name = "batched_decode" if args.workload == "default" else args.workload

    def counts(wname):
        K = args.steps if args.steps is not None else DEFAULT_STEPS[wname]
        Wm = args.warmup if args.warmup is not None else max(1, K // 50)
        return K, Wm

    def run(wname):
        K, Wm = counts(wname)
        wl = make_workload(wname, args)
        return measure(wl, wname, K, Wm, max(3, min(200, K // wl.R)), args.cpu_budget, stream)

    K, Wm = counts(name)
    head = run(name)
    line = {"metric": METRIC, "value": head.pop("value"), "unit": "tokens/s", "n_gpus": 1,
            "steps": K, "warmup": Wm, "ms_per_step": head.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": head.pop("dtype"), "data": "synthetic"}
    head.pop("steps")
    head.pop("warmup")
    line.update(head)
    if args.workload == "default":
        torch.cuda.empty_cache()
        line["prefill"] = {"workload": "mixed_prefill", **run("mixed_prefill")}
        torch.cuda.empty_cache()
        m = machine_reference(stream, line["prefill"]["roofline"]["bytes_per_launch"])
        if m is not None:
            # the kernels against what this GPU reaches on their patterns
            line["roofline"]["floor_us"] = m["decode_chain_floor_us"]
            line["roofline"]["launch_over_floor"] = round(
                line["roofline"]["launch_us"] / m["decode_chain_floor_us"], 3)
            pr = line["prefill"]["roofline"]
            # the best this GPU reached on the prefill's traffic: the pattern
            # at either size, or the launch's own layout
            pr["ceiling_GBs"] = round(max(m["prefill_pattern_TBs"],
                                          m["prefill_pattern_at_launch_size_TBs"],
                                          m["prefill_layout_TBs"]) * 1e3, 1)
            pr["frac_of_ceiling"] = round(pr["achieved"] / pr["ceiling_GBs"], 4)
        line["machine"] = m
    line["kernel_sources"] = kernel_source_digest()
    if OTHER_LIB:
        line["library"] = OTHER_LIB
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
