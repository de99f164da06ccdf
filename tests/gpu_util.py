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


def dtype_name(t: torch.dtype) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t]


def live_rows(case) -> np.ndarray:
    return to_np(case.slot_mapping) >= 0
