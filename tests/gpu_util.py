"""Runners shared by the GPU parity tests, the smoke check and the bench:
one for the HIP library (through its C ABI binding) and one for the oracle,
fed the same generator inputs."""
from __future__ import annotations

import numpy as np
import torch

from tests.helpers import to_np

SENTINEL = -777.0


def gpu_fused(case, dev="cuda", out_init=None, fold=False):
    """Run metadata + fused insert/conv on the GPU (or, with fold=True, the
    single launch that searches query_start_loc itself).  Returns device
    tensors (out, cache, seq_idx, query_start) -- the last two None when
    folded; the case's cache is not modified."""
    import depthwise_causal_conv1d_amd as lib
    T = case.T
    x = case.x.to(dev)
    w = case.weight.to(dev)
    cache = case.cache.to(dev).clone()
    pos = case.positions.to(dev)
    bt = case.block_table.to(dev)
    sm = case.slot_mapping.to(dev)
    qsl = case.query_start_loc.to(dev)
    out = (torch.full_like(x, SENTINEL) if out_init is None else out_init.to(dev).clone())
    if fold:
        lib.sconv_fused_insert_conv_qsl(x, w, cache, pos, bt, qsl, case.num_reqs, sm, case.off_s,
                                        case.ws, case.block_size, case.activation,
                                        case.use_residual, out=out)
        return out, cache, None, None
    seq_idx = torch.full((T,), -5, dtype=torch.int32, device=dev)
    qs = torch.full((T,), -5, dtype=torch.int32, device=dev)
    lib.sconv_seq_metadata(qsl, case.num_reqs, case.num_actual, seq_idx, qs, T)
    lib.sconv_fused_insert_conv(x, w, cache, pos, bt, seq_idx, sm, qs, case.off_s, case.ws,
                                case.block_size, case.activation, case.use_residual, out=out)
    return out, cache, seq_idx, qs


def gpu_plan(case, dev="cuda"):
    """The launch gpu_fused(case) makes for its fused call (per-row
    request buffers), as sconv_fused_plan's dict; nothing is launched."""
    import depthwise_causal_conv1d_amd as lib
    seq_idx = torch.zeros(case.T, dtype=torch.int32, device=dev)
    return lib.sconv_fused_plan([case.x.to(dev)], [case.weight.to(dev)], case.cache.to(dev),
                                case.positions.to(dev), case.block_table.to(dev),
                                case.slot_mapping.to(dev), [case.off_s], [case.ws],
                                case.block_size, case.activation, case.use_residual,
                                seq_idx=seq_idx, query_start=seq_idx.clone())


def oracle_fused(case, cache=None, block_table=None, slot_mapping=None, out_init=None):
    """The oracle on the same inputs (optionally a compacted cache)."""
    import oracle
    si, qs = oracle.seq_metadata(to_np(case.query_start_loc), case.num_reqs, case.num_actual,
                                 case.T)
    if out_init is None:
        out_init = torch.full_like(case.x, SENTINEL)
    out, cache_after = oracle.fused_insert_conv(
        to_np(case.x), to_np(case.weight), to_np(case.cache if cache is None else cache),
        to_np(case.positions), to_np(case.block_table if block_table is None else block_table),
        si, to_np(case.slot_mapping if slot_mapping is None else slot_mapping), qs,
        case.off_s, case.ws, case.block_size, case.activation, case.use_residual,
        out_init=to_np(out_init))
    return out, cache_after, si, qs


def gpu_fused_streams(cases, dev="cuda", fold=True):
    """All streams of ``cases`` (one layer, shared cache) in one
    sconv_fused_insert_conv_streams launch; rows find their request inside
    the launch (fold) or from sconv_seq_metadata buffers.  Returns (outs,
    cache) as device tensors; the cases are not modified."""
    import depthwise_causal_conv1d_amd as lib
    c0 = cases[0]
    xs = [c.x.to(dev) for c in cases]
    ws_ = [c.weight.to(dev) for c in cases]
    cache = c0.cache.to(dev).clone()
    pos = c0.positions.to(dev)
    bt = c0.block_table.to(dev)
    sm = c0.slot_mapping.to(dev)
    qsl = c0.query_start_loc.to(dev)
    outs = [torch.full_like(x, SENTINEL) for x in xs]
    kw = dict(activation=[c.activation for c in cases],
              use_residual=[c.use_residual for c in cases], outs=outs)
    if fold:
        kw.update(query_start_loc=qsl, num_reqs=c0.num_reqs)
    else:
        si = torch.full((c0.T,), -5, dtype=torch.int32, device=dev)
        qs = torch.full((c0.T,), -5, dtype=torch.int32, device=dev)
        lib.sconv_seq_metadata(qsl, c0.num_reqs, c0.num_actual, si, qs, c0.T)
        kw.update(seq_idx=si, query_start=qs)
    lib.sconv_fused_insert_conv_streams(xs, ws_, cache, pos, bt, sm, [c.off_s for c in cases],
                                        [c.ws for c in cases], c0.block_size, **kw)
    return outs, cache


def oracle_fused_streams(cases, cache=None, block_table=None, slot_mapping=None):
    """The oracle's multi-stream op on the same inputs (optionally a
    compacted cache).  Returns (outs, cache_after)."""
    import oracle
    c0 = cases[0]
    si, qs = oracle.seq_metadata(to_np(c0.query_start_loc), c0.num_reqs, c0.num_actual, c0.T)
    specs = [{"x": to_np(c.x), "weight": to_np(c.weight), "off_s": c.off_s, "ws": c.ws,
              "activation": c.activation, "use_residual": c.use_residual,
              "out_init": to_np(torch.full_like(c.x, SENTINEL))} for c in cases]
    return oracle.fused_insert_conv_streams(
        specs, to_np(c0.cache if cache is None else cache), to_np(c0.positions),
        to_np(c0.block_table if block_table is None else block_table), si,
        to_np(c0.slot_mapping if slot_mapping is None else slot_mapping), qs, c0.block_size)


def dtype_name(t: torch.dtype) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t]


def live_rows(case) -> np.ndarray:
    return to_np(case.slot_mapping) >= 0


def written_cache_values(cache: np.ndarray, slot_mapping: np.ndarray, block_size: int,
                         off_s: int, ws: int) -> np.ndarray:
    """The cache columns [off_s, off_s + ws) of every head at the slots of
    the non-PAD rows: what an insert writes."""
    sm = np.asarray(slot_mapping)
    live = sm[sm >= 0]
    return cache[live // block_size, :, live % block_size, off_s:off_s + ws]
