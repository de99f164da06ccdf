"""Benchmark of the paged short-convolution hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline): batched decode -- 256 requests x 1 token,
history lengths uniform in [1, 4096], H=32, D=128, ws=32 (C=1024), W=4,
N=16, bf16, SiLU and residual.  One step is one pass of the hot path over one
decode batch, replayed from a hipGraph: by default one launch of
sconv_fused_insert_conv_qsl (request search, insert and conv);
`--metadata separate` runs sconv_seq_metadata + sconv_fused_insert_conv.
Other workloads (same JSON shape, one line each):
  decode_layer      the decode batch with all four streams of a layer
                    (ws=32 each) in one sconv_fused_insert_conv_streams launch
  mixed_prefill     16 requests, ~17-20k rows, 4 streams of C=4096 over one
                    cache, 10% PAD rows; step = metadata + 4 fused launches
  spec_decode       512 requests x 4 draft rows, C=4096, N=32; step = folded
                    fused launch + conv-window gather (device real_count)
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

Prints one JSON line.  `value` is tokens per second over the K timed steps
(wall clock between two device synchronizations).  `roofline` describes the
workload's dominant kernel: algorithmic bytes per launch divided by its
average launch duration, timed with HIP events on the stream it runs on.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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


def kernel_source_digest() -> str:
    """Hash of the GPU sources without their comments, to tell whether
    stored counters were taken on the kernels as they are now."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current sources."""
    path = os.path.join(PROFILES, f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_sources:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest():
        return None
    return float(t.group(1))


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


def sub_case(case, rows, reqs, poison):
    """The requests `reqs` (rows `rows`) of a multi-batch case as a case of
    their own, for the oracle."""
    import torch

    import workloads
    bt = case.block_table[reqs]
    u = torch.unique(bt.long())
    if not (u == poison).any():
        u = torch.cat([u, torch.tensor([poison])])
    qsl = case.query_start_loc[reqs.start:reqs.stop + 1] - case.query_start_loc[reqs.start]
    return workloads.FusedCase(**{**case.__dict__, "x": case.x[rows],
                                  "positions": case.positions[rows], "block_table": bt,
                                  "slot_mapping": case.slot_mapping[rows],
                                  "query_start_loc": qsl.to(torch.int32),
                                  "num_reqs": reqs.stop - reqs.start,
                                  "num_actual": rows.stop - rows.start,
                                  "used_blocks": torch.sort(u).values})


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


def time_oracle_fused(case, activation="silu"):
    """Seconds the oracle spends on one fused launch of `case` (compact cache)."""
    import oracle
    from tests.helpers import to_np
    cache, bt, sm = case.compact()
    si, qs = oracle.seq_metadata(to_np(case.query_start_loc), case.num_reqs, case.num_actual,
                                 case.T)
    args = (to_np(case.x), to_np(case.weight), to_np(cache), to_np(case.positions), to_np(bt),
            si, to_np(sm), qs, case.off_s, case.ws, case.block_size, activation,
            case.use_residual)
    t0 = time.perf_counter()
    oracle.fused_insert_conv(*args)
    return time.perf_counter() - t0


# ---------------------------------------------------------------- workloads

class Workload:
    kernel_name = "fused_insert_conv_kernel"
    bound = "hbm"
    dtype = "bf16"

    def kernel(self, i):          # the dominant kernel alone
        raise NotImplementedError

    def kernels_per_call(self):   # launches of it per kernel(i)
        return 1


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

    def config(self):
        return {"workload": "batched_decode", "requests": self.B, "tokens_per_step": self.B,
                "metadata": "folded into the fused launch" if self.fold else "separate launch",
                "history": "uniform[1,4096]", "H": 32, "D": 128, "ws": 32, "C": 1024,
                "W": 4, "block_size": 16, "activation": "silu", "residual": True,
                "graph": "hipGraph", "replicas": self.R}

    def oracle_sample(self, budget):
        # Whole sub-batches of 256 requests, cycled, until the budget is spent.
        n_sub = self.R * self.B // 256

        def once(n):
            rows = slice(256 * (n % n_sub), 256 * (n % n_sub + 1))
            return 256, time_oracle_fused(sub_case(self.case, rows, rows, self.case.poison_block))
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

    def config(self):
        return {"workload": "decode_layer", "requests": self.B, "tokens_per_step": self.B,
                "streams": 4, "stream_launches": "one launch for all 4 streams"
                if self.one_launch else "one launch per stream",
                "metadata": "folded into the fused launch", "history": "uniform[1,4096]",
                "H": 32, "D": 128, "ws": 32, "C_per_stream": 1024, "W": 4, "block_size": 16,
                "activation": "silu", "residual": True, "graph": "hipGraph", "replicas": self.R}

    def oracle_sample(self, budget):
        # Whole sub-batches of 256 requests x 4 streams, cycled, until the
        # budget is spent.
        n_sub = self.R * self.B // 256

        def once(n):
            rows = slice(256 * (n % n_sub), 256 * (n % n_sub + 1))
            return 256, sum(time_oracle_fused(sub_case(k, rows, rows, k.poison_block))
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

    def oracle_sample(self, budget):
        # Whole streams (all rows), in turn, until the budget is spent; a
        # token counts once for its four streams.
        done, spent, n = repeat_until(
            budget, lambda n: (self.live / 4, time_oracle_fused(self.streams[n % 4])))
        return done / spent, f"{n} whole-stream passes over all {self.live} live rows", spent


class SpecDecodeBench(Workload):
    """Speculative decode (512 x 4 drafts) plus the conv-window gather."""

    B = 2048

    def __init__(self, dev="cuda", fold: bool = False):
        import torch

        import depthwise_causal_conv1d_amd as lib
        import workloads
        self.lib = lib
        self.fold = fold
        first = workloads.spec_decode()
        self.bytes_per_launch = fused_algorithmic_bytes(first)
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
        self.rc = torch.tensor([gc.real_count], dtype=torch.int32, device=dev)
        self.gout = torch.empty(self.R, 512, c.C, 3, dtype=torch.bfloat16, device=dev)
        self.real_count = gc.real_count
        self.tokens_per_step = self.B

    def rows(self, i):
        return slice(i * self.B, (i + 1) * self.B)

    def kernel(self, i):
        s, c = self.rows(i), self.case
        bt = self.bt[512 * i:512 * (i + 1)]
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
        self.lib.gather_intermediate_conv_window(self.x[self.rows(i)].view(1, self.B, -1),
                                                 self.gpos, self.rc, self.gout[i], 3)

    def config(self):
        return {"workload": "spec_decode", "requests": 512, "drafts": 4, "tokens_per_step": 2048,
                "metadata": "folded into the fused launch" if self.fold else "separate launch",
                "positions": "uniform[1,131072)", "H": 64, "D": 64, "ws": 64, "C": 4096,
                "W": 4, "block_size": 32, "gather": {"max_count": 512, "d_conv": 3,
                                                     "real_count": self.real_count},
                "activation": "silu", "residual": True, "graph": "hipGraph",
                "replicas": self.R}

    def oracle_sample(self, budget):
        def once(n):
            i = n % self.R
            sub = sub_case(self.case, self.rows(i), slice(512 * i, 512 * (i + 1)),
                           self.case.poison_block)
            return self.B, time_oracle_fused(sub)
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

    def oracle_sample(self, budget):
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
                                            ci[keep], hi[keep], "silu", -1)
            return 2 * L, time.perf_counter() - t0
        done, spent, n = repeat_until(budget, once)
        return (done / spent, f"{n} pairs of 4096-token sequences, one with a state and one "
                f"without ({done} tokens, all channels)", spent)


class SsmDecodeBench(Workload):
    kernel_name = "update_kernel"

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

    def oracle_sample(self, budget):
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

    def oracle_sample(self, budget):
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
    kernel_name = "gather_ssm_kernel"
    dtype = "f32"
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

    def oracle_sample(self, budget):
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

def capture(fn, indices):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in indices:
            fn(i)
    return g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="batched_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the CPU baseline (0: skip)")
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
    fold = (args.metadata == "folded" or
            (args.metadata == "auto" and args.workload in ("batched_decode", "spec_decode")))
    one = (args.stream_launches == "one" or
           (args.stream_launches == "auto" and args.workload == "decode_layer"))
    if args.workload == "batched_decode":
        wl = DecodeBench(requests=args.requests, fold=fold)
    elif args.workload == "decode_layer":
        wl = DecodeLayerBench(requests=args.requests, one_launch=one)
    elif args.workload == "mixed_prefill":
        wl = MixedPrefillBench(fold=fold, one_launch=one)
    elif args.workload == "spec_decode":
        wl = WORKLOADS[args.workload](fold=fold)
    else:
        wl = WORKLOADS[args.workload]()
    R = wl.R
    K = args.steps if args.steps is not None else DEFAULT_STEPS[args.workload]
    Wm = args.warmup if args.warmup is not None else max(R, K // 50)

    # Touch every replica once eagerly, then capture on a side stream.
    for i in range(R):
        wl.step(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g_all = capture(wl.step, range(R))
        rem = K % R
        g_rem = capture(wl.step, range(rem)) if rem else None
        g_kern = capture(wl.kernel, range(R))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def run_steps(n):
        for _ in range(n // R):
            g_all.replay()
        if n % R:
            g_rem.replay()

    run_steps(Wm - Wm % R if Wm >= R else R)
    torch.cuda.synchronize()

    # Timed region: exactly K steps.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(K)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Average duration of one launch of the dominant kernel: graphs holding
    # only that kernel (R calls per replay), bracketed by HIP events on the
    # stream the kernels run on.
    reps = max(3, min(200, K // R))
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(reps):
        g_kern.replay()
    k1.record(stream)
    torch.cuda.synchronize()
    launches = reps * R * wl.kernels_per_call()
    kern_us = k0.elapsed_time(k1) * 1e3 / launches
    achieved = wl.bytes_per_launch / (kern_us * 1e-6) / 1e9

    cpu = None
    if args.cpu_budget > 0:
        v, sample, spent = wl.oracle_sample(args.cpu_budget)
        cpu = {"value": round(v, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{sample}; {spent:.1f} s single-threaded"}

    traffic = stored_traffic(args.workload)
    value = wl.tokens_per_step * K / wall
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(wall * 1e3 / K, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": wl.config(),
        "roofline": {"bound": wl.bound, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": wl.kernel_name,
                     "bytes_per_launch": wl.bytes_per_launch, "launch_us": round(kern_us, 3)},
        "cpu_baseline": cpu,
        "kernel_sources": kernel_source_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
