"""Seeded synthetic inputs for the paged short-convolution ops.

This module only draws and lays out inputs: request lengths, positions, block
tables, slot mappings, PAD rows, input rows, weights and cache contents.  It
holds none of the convolution's arithmetic, so that both the oracle and the
GPU path can be fed from it.

Conventions shared by every generator:
  * all draws come from one ``torch.Generator`` seeded by ``seed`` on the CPU,
    in the fixed order written in each function;
  * bfloat16 values are float32 draws rounded by ``Tensor.to(bfloat16)``, so
    every consumer sees the same bits;
  * cache positions the op must never read hold NaN ("poison"); so do
    block-table entries that no request owns (they point at a poison block).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dt(dtype):
    return DTYPES[dtype] if isinstance(dtype, str) else dtype


@dataclass
class FusedCase:
    """Inputs of one insert + conv launch over a paged cache (one stream)."""
    x: torch.Tensor              # [T, H*ws]
    weight: torch.Tensor         # [H*ws, W]
    cache: torch.Tensor          # [num_blocks, H, N, D] (may live on a GPU)
    positions: torch.Tensor      # int64 [T]
    block_table: torch.Tensor    # int32 [num_reqs, max_blocks]
    slot_mapping: torch.Tensor   # int64 [T], -1 = PAD
    query_start_loc: torch.Tensor  # int32 [num_reqs + 1]
    num_reqs: int
    num_actual: int              # rows covered by requests
    off_s: int
    ws: int
    block_size: int
    W: int
    activation: Optional[str]
    use_residual: bool
    used_blocks: torch.Tensor    # int64 physical ids referenced by block_table
    poison_block: int

    @property
    def T(self) -> int:
        return self.x.shape[0]

    @property
    def H(self) -> int:
        return self.cache.shape[1]

    @property
    def C(self) -> int:
        return self.x.shape[1]

    def select(self, rows: slice, reqs: slice) -> "FusedCase":
        """Requests ``reqs`` (whose rows are ``rows``) of a multi-batch case
        as a case of their own: their rows, block-table rows and request
        offsets (rebased to 0), over the same cache."""
        bt = self.block_table[reqs]
        u = torch.unique(bt.long())
        if not (u == self.poison_block).any():
            u = torch.cat([u, torch.tensor([self.poison_block])])
        qsl = self.query_start_loc[reqs.start:reqs.stop + 1] - self.query_start_loc[reqs.start]
        return FusedCase(**{**self.__dict__, "x": self.x[rows],
                            "positions": self.positions[rows], "block_table": bt,
                            "slot_mapping": self.slot_mapping[rows],
                            "query_start_loc": qsl.to(torch.int32),
                            "num_reqs": reqs.stop - reqs.start,
                            "num_actual": rows.stop - rows.start,
                            "used_blocks": torch.sort(u).values})

    def compact(self):
        """(cache, block_table, slot_mapping) restricted to the referenced
        blocks, renumbered 0..n-1: the same logical content in a small host
        array, for consumers that cannot hold the whole pool."""
        ids = self.used_blocks
        remap = torch.full((self.cache.shape[0],), -1, dtype=torch.int64)
        remap[ids] = torch.arange(ids.numel(), dtype=torch.int64)
        cache = self.cache[ids.to(self.cache.device)].cpu()
        bt = remap[self.block_table.long()].to(torch.int32)
        sm = self.slot_mapping.clone()
        live = sm >= 0
        N = self.block_size
        sm[live] = remap[sm[live] // N] * N + sm[live] % N
        return cache, bt, sm


def fused_case(seed: int, new_lens: List[int], ctx_lens: List[int], *, H: int, D: int,
               ws: int, off_s: int = 0, block_size: int = 16, W: int = 4, dtype="bf16",
               pad_count: int = 0, tail_pad: int = 0, pool_blocks: Optional[int] = None,
               activation: Optional[str] = "silu", use_residual: bool = True,
               zero_cache: bool = False, w_std: float = 0.5, device="cpu",
               x: Optional[torch.Tensor] = None, weight: Optional[torch.Tensor] = None,
               gen: Optional[torch.Generator] = None) -> FusedCase:
    """Requests r = 0..R-1 bring ``new_lens[r]`` new tokens at positions
    ``ctx_lens[r] .. ctx_lens[r]+new_lens[r]-1`` (their rows are packed in
    request order), after ``ctx_lens[r]`` tokens already in the cache.

    Draw order: x, weight, physical block permutation, history rows, PAD rows.
    Blocks are allocated for the sliding window each request touches, that is
    the positions from ``ctx - (W-1)`` to its last new token; every other
    block-table entry points at a poison block.  ``tail_pad`` extra rows at
    the end have slot -1 (padding up to a captured token count).
    """
    dt = _dt(dtype)
    g = gen if gen is not None else torch.Generator().manual_seed(seed)
    R = len(new_lens)
    assert len(ctx_lens) == R and all(n >= 0 for n in new_lens) and all(c >= 0 for c in ctx_lens)
    N = block_size
    C = H * ws
    T_act = int(sum(new_lens))
    T = T_act + tail_pad

    # 1. input rows and weights
    if x is None:
        x = torch.randn(T, C, generator=g).to(dt)
    if weight is None:
        weight = (torch.randn(C, W, generator=g) * w_std).to(dt)

    # 2. packing: request rows are contiguous, positions consecutive
    qsl = torch.zeros(R + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(new_lens, dtype=torch.int64), 0).to(torch.int32)
    positions = torch.zeros(T, dtype=torch.int64)
    req_of_row = torch.zeros(T_act, dtype=torch.int64)
    for r in range(R):
        a, b = int(qsl[r]), int(qsl[r + 1])
        positions[a:b] = torch.arange(ctx_lens[r], ctx_lens[r] + new_lens[r])
        req_of_row[a:b] = r

    # 3. blocks: the window each request touches
    spans = []
    max_blocks = 1
    for r in range(R):
        lo = max(0, ctx_lens[r] - (W - 1))
        hi = ctx_lens[r] + new_lens[r] - 1
        if hi < lo:           # nothing new and nothing to read
            spans.append(range(0))
            continue
        spans.append(range(lo // N, hi // N + 1))
        max_blocks = max(max_blocks, hi // N + 1)
    needed = sum(len(s) for s in spans)
    pool = pool_blocks if pool_blocks is not None else needed + 1
    assert pool >= needed + 1, "pool must hold every touched block plus a poison block"
    perm = torch.randperm(pool, generator=g)
    poison = int(perm[needed])
    block_table = torch.full((R, max_blocks), poison, dtype=torch.int32)
    k = 0
    used = []
    for r, s in enumerate(spans):
        for lb in s:
            block_table[r, lb] = int(perm[k])
            used.append(int(perm[k]))
            k += 1
    used.append(poison)
    used_blocks = torch.tensor(sorted(set(used)), dtype=torch.int64)

    # 4. slot of each real row: its position's cache cell
    slot_mapping = torch.full((T,), -1, dtype=torch.int64)
    if T_act:
        p = positions[:T_act]
        blk = block_table[req_of_row, p // N].long()
        slot_mapping[:T_act] = blk * N + p % N

    # 5. cache: poison everywhere except the history rows the window reads
    if zero_cache:
        cache = torch.zeros(pool, H, N, D, dtype=dt, device=device)
    else:
        cache = torch.full((pool, H, N, D), float("nan"), dtype=dt, device=device)
    hist = []
    for r in range(R):
        for pos in range(max(0, ctx_lens[r] - (W - 1)), ctx_lens[r]):
            hist.append((int(block_table[r, pos // N]), pos % N))
    if hist:
        vals = torch.randn(len(hist), H, D, generator=g).to(dt)
        if zero_cache:
            vals.zero_()
        bi = torch.tensor([h[0] for h in hist], dtype=torch.int64)
        oi = torch.tensor([h[1] for h in hist], dtype=torch.int64)
        cache[bi.to(device), :, oi.to(device), :] = vals.to(device)

    # 6. PAD rows among the real rows (exact count)
    if pad_count:
        pads = torch.randperm(T_act, generator=g)[:pad_count]
        slot_mapping[pads] = -1

    return FusedCase(x=x, weight=weight, cache=cache, positions=positions,
                     block_table=block_table, slot_mapping=slot_mapping,
                     query_start_loc=qsl, num_reqs=R, num_actual=T_act, off_s=off_s, ws=ws,
                     block_size=N, W=W, activation=activation, use_residual=use_residual,
                     used_blocks=used_blocks, poison_block=poison)


def fused_streams_case(seed: int, new_lens: List[int], ctx_lens: List[int], *, H: int, D: int,
                       streams, block_size: int = 16, W: int = 4, dtype="bf16",
                       pad_count: int = 0, tail_pad: int = 0,
                       pool_blocks: Optional[int] = None, activations=None, residuals=None,
                       device="cpu") -> List[FusedCase]:
    """Several conv streams of one layer over one shared cache: ``streams``
    lists (off_s, ws) per stream.  Stream 0 is ``fused_case`` with these
    arguments; each further stream draws its own x [T, H*ws] and weight
    [H*ws, W] (N(0,1), N(0,0.5)) from a second generator seeded seed + 7919,
    in stream order.  ``activations`` / ``residuals`` give one value per
    stream (default SiLU and residual for all)."""
    dt = _dt(dtype)
    off0, ws0 = streams[0]
    acts = activations if activations is not None else ["silu"] * len(streams)
    ress = residuals if residuals is not None else [True] * len(streams)
    base = fused_case(seed, new_lens, ctx_lens, H=H, D=D, ws=ws0, off_s=off0,
                      block_size=block_size, W=W, dtype=dtype, pad_count=pad_count,
                      tail_pad=tail_pad, pool_blocks=pool_blocks, activation=acts[0],
                      use_residual=ress[0], device=device)
    g = torch.Generator().manual_seed(seed + 7919)
    cases = [base]
    for k, (off, ws) in enumerate(streams[1:], start=1):
        x = torch.randn(base.T, H * ws, generator=g).to(dt)
        w = (torch.randn(H * ws, W, generator=g) * 0.5).to(dt)
        cases.append(FusedCase(**{**base.__dict__, "x": x, "weight": w, "off_s": off, "ws": ws,
                                  "activation": acts[k], "use_residual": ress[k]}))
    return cases


# ---------------------------------------------------------------- SSM-style ops

@dataclass
class VarlenCase:
    x: torch.Tensor                # [dim, total_T] channel-major
    weight: torch.Tensor           # [dim, W]
    bias: Optional[torch.Tensor]   # [dim]
    conv_states: torch.Tensor      # [num_slots, dim, W-1]
    query_start_loc: torch.Tensor  # int32 [batch+1]
    cache_indices: Optional[torch.Tensor]  # int32 [batch]
    has_initial_state: Optional[torch.Tensor]  # bool [batch]
    activation: Optional[str]
    pad_slot_id: int
    W: int


def varlen_case(seed: int, seq_lens: List[int], *, dim: int, num_slots: int, W: int = 4,
                dtype="bf16", init_count: Optional[int] = None, pad_seqs: int = 0,
                bias_std: Optional[float] = 0.1, w_std: float = 0.5,
                activation: Optional[str] = "silu", pad_slot_id: int = -1,
                x_padding: int = 0, device="cpu") -> VarlenCase:
    """Sequences b = 0..batch-1 of lengths ``seq_lens`` packed along tokens.

    Draw order: x, weight, bias, slot permutation, initial-state choice,
    initial states, PAD choice.  Slots without an initial state hold NaN.
    ``x_padding`` widens the channel stride of x beyond total_T.
    """
    dt = _dt(dtype)
    g = torch.Generator().manual_seed(seed)
    B = len(seq_lens)
    total = int(sum(seq_lens))
    xb = torch.randn(dim, total + x_padding, generator=g).to(dt)
    x = xb[:, :total] if x_padding else xb
    weight = (torch.randn(dim, W, generator=g) * w_std).to(dt)
    bias = (torch.randn(dim, generator=g) * bias_std).to(dt) if bias_std is not None else None
    assert num_slots >= B
    cache_indices = torch.randperm(num_slots, generator=g)[:B].to(torch.int32)
    if init_count is None:
        init_count = B // 2
    has_init = torch.zeros(B, dtype=torch.bool)
    has_init[torch.randperm(B, generator=g)[:init_count]] = True
    conv_states = torch.full((num_slots, dim, W - 1), float("nan"), dtype=dt, device=device)
    n_init = int(has_init.sum())
    if n_init:
        vals = torch.randn(n_init, dim, W - 1, generator=g).to(dt)
        conv_states[cache_indices[has_init].long().to(device)] = vals.to(device)
    if pad_seqs:
        pads = torch.randperm(B, generator=g)[:pad_seqs]
        cache_indices[pads] = pad_slot_id
    qsl = torch.zeros(B + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(seq_lens, dtype=torch.int64), 0).to(torch.int32)
    return VarlenCase(x=x, weight=weight, bias=bias, conv_states=conv_states,
                      query_start_loc=qsl, cache_indices=cache_indices,
                      has_initial_state=has_init, activation=activation,
                      pad_slot_id=pad_slot_id, W=W)


def update_inputs(seed: int, steps: int, batch: int, dim: int, dtype="bf16") -> List[torch.Tensor]:
    """``steps`` decode inputs x_s [batch, dim] drawn N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(batch, dim, generator=g).to(_dt(dtype)) for _ in range(steps)]


@dataclass
class GatherCase:
    src: torch.Tensor              # [1, seq_len, conv_dim]
    abs_positions: torch.Tensor    # int32 [max_count]
    real_count: int
    out_init: torch.Tensor         # [max_count, conv_dim, d_conv] sentinel-filled
    d_conv: int


def gather_case(seed: int, src: torch.Tensor, *, max_count: int, d_conv: int,
                stride: int = 4, real_count: Optional[int] = None,
                sentinel: float = -777.0) -> GatherCase:
    """Slot i extracts the window ending at ``stride*i + a_i``, a_i uniform
    in [1, stride]; ``real_count`` uniform in [0, max_count] unless given."""
    g = torch.Generator().manual_seed(seed)
    a = torch.randint(1, stride + 1, (max_count,), generator=g)
    pos = (torch.arange(max_count) * stride + a).to(torch.int32)
    if real_count is None:
        real_count = int(torch.randint(0, max_count + 1, (1,), generator=g))
    conv_dim = src.shape[-1]
    out = torch.full((max_count, conv_dim, d_conv), sentinel, dtype=src.dtype)
    return GatherCase(src=src, abs_positions=pos, real_count=real_count, out_init=out,
                      d_conv=d_conv)


# ---------------------------------------------------------------- named workloads

def tiny_prefill(device="cpu") -> FusedCase:
    """One request, 64 new tokens at positions 0..63, H=2, ws=8 (C=16), D=32,
    N=16, fp32, zero cache of 8 blocks, SiLU and residual, seed 0."""
    return fused_case(0, [64], [0], H=2, D=32, ws=8, off_s=0, block_size=16, W=4,
                      dtype="f32", pool_blocks=8, zero_cache=True, device=device)


def _uniform_ints(g, lo, hi, n):
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=g)]


def batched_decode(device="cpu", num_reqs: int = 256, seed: int = 1,
                   pool_blocks: Optional[int] = None) -> FusedCase:
    """num_reqs requests x 1 token; history lengths uniform in [1, 4096];
    H=32, D=128, ws=32 (C=1024), W=4, N=16, bf16, SiLU, residual."""
    g = torch.Generator().manual_seed(seed)
    ctx = _uniform_ints(g, 1, 4096, num_reqs)
    return fused_case(seed, [1] * num_reqs, ctx, H=32, D=128, ws=32, off_s=0, block_size=16,
                      W=4, dtype="bf16", pool_blocks=pool_blocks, device=device, gen=g)


def mixed_prefill_streams(device="cpu", seed: int = 2) -> List[FusedCase]:
    """16 requests, new lengths uniform in [128, 2048]; 8 of them (random)
    carry a cached prefix uniform in [0, 8192].  H=32, D=512 split into four
    streams ws=128 at off_s 0/128/256/384, each with its own x and weight,
    one shared cache; 10% of rows PAD.  bf16, SiLU, residual."""
    g = torch.Generator().manual_seed(seed)
    R = 16
    new = _uniform_ints(g, 128, 2048, R)
    with_ctx = torch.randperm(R, generator=g)[: R // 2]
    ctx = [0] * R
    for r in with_ctx.tolist():
        ctx[r] = int(torch.randint(0, 8193, (1,), generator=g))
    T = sum(new)
    base = fused_case(seed, new, ctx, H=32, D=512, ws=128, off_s=0, block_size=16, W=4,
                      dtype="bf16", pad_count=T // 10, device=device, gen=g)
    cases = [base]
    for s in range(1, 4):
        xs = torch.randn(T, 32 * 128, generator=g).to(torch.bfloat16)
        wsd = (torch.randn(32 * 128, 4, generator=g) * 0.5).to(torch.bfloat16)
        cases.append(FusedCase(**{**base.__dict__, "x": xs, "weight": wsd, "off_s": 128 * s}))
    return cases


def ssm_varlen(device="cpu", seed: int = 3, seqs: int = 8, seq_len: int = 4096,
               dim: int = 8192) -> VarlenCase:
    """8 sequences x 4096 tokens, dim 8192, W=4, bf16 channel-major, bias
    N(0, 0.1), pool of 1024 slots, half with an initial state, SiLU."""
    return varlen_case(seed, [seq_len] * seqs, dim=dim, num_slots=1024, W=4, dtype="bf16",
                       init_count=seqs // 2, device=device)


def spec_decode(device="cpu", seed: int = 4, num_reqs: int = 512,
                pool_blocks: Optional[int] = None) -> FusedCase:
    """num_reqs requests x 4 draft tokens at p..p+3, p uniform in
    [1, 131071]; H=64, ws=D=64 (C=4096), N=32, bf16, SiLU, residual."""
    g = torch.Generator().manual_seed(seed)
    ctx = _uniform_ints(g, 1, 131071 - 3, num_reqs)
    return fused_case(seed, [4] * num_reqs, ctx, H=64, D=64, ws=64, off_s=0, block_size=32,
                      W=4, dtype="bf16", pool_blocks=pool_blocks, device=device, gen=g)


def spec_gather(case: FusedCase, seed: int = 4, real_count: Optional[int] = None) -> GatherCase:
    """Windows of length 3 over the spec batch's inputs viewed [1, T, C],
    max_count 512."""
    return gather_case(seed + 1000, case.x.view(1, case.T, case.C), max_count=512, d_conv=3,
                       stride=4, real_count=real_count)
