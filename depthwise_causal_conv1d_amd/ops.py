"""Python binding of libsconv: torch tensors in, one C-ABI call out.

Each function only checks what the C ABI cannot see (tensor dtype, device,
dimensionality), turns tensors into pointers, element strides and the
current HIP stream, and calls the library.  All computation happens in the
HIP kernels; there is no CPU path.  Argument names follow the source pages.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib

_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"element type must be float32 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def _act(activation) -> int:
    if activation in (None, False, "none"):
        return _lib.ACT_NONE
    if activation in (True, "silu", "swish"):
        return _lib.ACT_SILU
    raise ValueError(f"unknown activation {activation!r}")


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libsconv tensors must live on the GPU")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _vec(t: torch.Tensor, dtype: torch.dtype, name: str, min_len: int = 0):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous 1-D tensor")
    if t.numel() < min_len:
        raise ValueError(f"{name} has {t.numel()} entries, needs {min_len}")


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def sconv_init() -> None:
    """Load the library's GPU code on the current device (before a first
    call that is captured into a graph)."""
    _lib.check(_lib.load().sconv_init(), "sconv_init")


def sconv_seq_metadata(query_start_loc: torch.Tensor, num_reqs: int, num_actual_tokens: int,
                       seq_idx_out: torch.Tensor, query_start_out: torch.Tensor,
                       num_padded_tokens: Optional[int] = None) -> None:
    """Fill the static per-token seq_idx / query_start buffers in one launch."""
    if num_padded_tokens is None:
        num_padded_tokens = num_actual_tokens
    _dev(query_start_loc, seq_idx_out, query_start_out)
    _vec(query_start_loc, torch.int32, "query_start_loc", num_reqs + 1 if num_actual_tokens else 0)
    _vec(seq_idx_out, torch.int32, "seq_idx_out")
    _vec(query_start_out, torch.int32, "query_start_out")
    rc = _lib.load().sconv_seq_metadata(
        _ptr(query_start_loc), int(num_reqs), int(num_actual_tokens), int(num_padded_tokens),
        _ptr(seq_idx_out), seq_idx_out.numel(), _ptr(query_start_out), query_start_out.numel(),
        _stream(seq_idx_out))
    _lib.check(rc, "sconv_seq_metadata")


def _fused_checks(x, weight, cache, positions, block_table, slot_mapping, off_s, ws,
                  block_size, out):
    T = x.shape[0]
    if x.dim() != 2 or weight.dim() != 2 or cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("x [T, C], weight [C, W], cache [nb, H, N, D], block_table [R, M]")
    if block_table.shape[1] > 1 and block_table.stride(1) != 1:
        # the C ABI takes a row stride only: entries of a row are contiguous
        raise ValueError("block_table needs contiguous entries within a row")
    _dev(x, weight, cache, positions, block_table, slot_mapping, out)
    dt = _dtype(x)
    if weight.dtype != x.dtype or cache.dtype != x.dtype or out.dtype != x.dtype:
        raise TypeError("x, weight, cache and out must share one element type")
    if x.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("x and out need contiguous channels")
    if cache.stride(3) != 1:
        raise ValueError("cache D-dim must be contiguous")
    nb, H, N, D = cache.shape
    if N != block_size:
        raise ValueError(f"block_size {block_size} != cache block dim {N}")
    if x.shape[1] != H * ws or weight.shape[0] != H * ws or out.shape != x.shape:
        raise ValueError("x / weight / out channel dim must be H*ws")
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be int32")
    _vec(positions, torch.int64, "positions", T)
    _vec(slot_mapping, torch.int64, "slot_mapping", T)
    return dt


def _table_rows(block_table: torch.Tensor, num_reqs: int):
    # With the request offsets the launch may read any row below num_reqs.
    if block_table.shape[0] < num_reqs:
        raise ValueError(f"block_table has {block_table.shape[0]} rows, needs num_reqs="
                         f"{num_reqs}")


def sconv_fused_insert_conv(x: torch.Tensor, weight: torch.Tensor, cache: torch.Tensor,
                            positions: torch.Tensor, block_table: torch.Tensor,
                            seq_idx: torch.Tensor, slot_mapping: torch.Tensor,
                            query_start: torch.Tensor, off_s: int, ws: int, block_size: int,
                            activation: Optional[str] = None, use_residual: bool = True,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Single-launch insert + depthwise causal conv1d over the paged cache.

    x [T, H*ws], weight [H*ws, W], cache [num_blocks, H, N, D] (modified),
    positions int64 [T], block_table int32 [num_reqs, max_blocks],
    seq_idx / query_start int32 [T], slot_mapping int64 [T] (-1 = PAD).
    Returns ``out`` (new [T, H*ws] tensor unless given; PAD rows untouched).
    """
    if out is None:
        out = torch.empty_like(x)
    if x.shape[0] == 0:
        return out
    dt = _fused_checks(x, weight, cache, positions, block_table, slot_mapping, off_s, ws,
                       block_size, out)
    T = x.shape[0]
    _dev(seq_idx, query_start)
    _vec(seq_idx, torch.int32, "seq_idx", T)
    _vec(query_start, torch.int32, "query_start", T)
    nb, H, N, D = cache.shape
    rc = _lib.load().sconv_fused_insert_conv(
        _ptr(x), x.stride(0), _ptr(weight), weight.stride(0), weight.stride(1),
        _ptr(cache), nb, H, N, D, cache.stride(0), cache.stride(1), cache.stride(2),
        _ptr(positions), _ptr(block_table), block_table.stride(0), block_table.shape[1],
        _ptr(seq_idx), _ptr(slot_mapping), _ptr(query_start), _ptr(out), out.stride(0),
        T, int(off_s), int(ws), weight.shape[1], dt, _act(activation), int(bool(use_residual)),
        _stream(x))
    _lib.check(rc, "sconv_fused_insert_conv")
    return out


def sconv_fused_insert_conv_qsl(x: torch.Tensor, weight: torch.Tensor, cache: torch.Tensor,
                                positions: torch.Tensor, block_table: torch.Tensor,
                                query_start_loc: torch.Tensor, num_reqs: int,
                                slot_mapping: torch.Tensor, off_s: int, ws: int,
                                block_size: int, activation: Optional[str] = None,
                                use_residual: bool = True,
                                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sconv_seq_metadata + sconv_fused_insert_conv in one launch: rows find
    their request in query_start_loc [num_reqs + 1] inside the kernel."""
    if out is None:
        out = torch.empty_like(x)
    if x.shape[0] == 0:
        return out
    dt = _fused_checks(x, weight, cache, positions, block_table, slot_mapping, off_s, ws,
                       block_size, out)
    T = x.shape[0]
    _dev(query_start_loc)
    _vec(query_start_loc, torch.int32, "query_start_loc", num_reqs + 1)
    _table_rows(block_table, num_reqs)
    nb, H, N, D = cache.shape
    rc = _lib.load().sconv_fused_insert_conv_qsl(
        _ptr(x), x.stride(0), _ptr(weight), weight.stride(0), weight.stride(1),
        _ptr(cache), nb, H, N, D, cache.stride(0), cache.stride(1), cache.stride(2),
        _ptr(positions), _ptr(block_table), block_table.stride(0), block_table.shape[1],
        _ptr(query_start_loc), int(num_reqs), _ptr(slot_mapping), _ptr(out), out.stride(0),
        T, int(off_s), int(ws), weight.shape[1], dt, _act(activation), int(bool(use_residual)),
        _stream(x))
    _lib.check(rc, "sconv_fused_insert_conv_qsl")
    return out


def sconv_fused_insert_conv_streams(xs: Sequence[torch.Tensor], weights: Sequence[torch.Tensor],
                                    cache: torch.Tensor, positions: torch.Tensor,
                                    block_table: torch.Tensor, slot_mapping: torch.Tensor,
                                    off_s: Sequence[int], ws: Sequence[int], block_size: int,
                                    activation=None, use_residual=True,
                                    seq_idx: Optional[torch.Tensor] = None,
                                    query_start: Optional[torch.Tensor] = None,
                                    query_start_loc: Optional[torch.Tensor] = None,
                                    num_reqs: Optional[int] = None,
                                    outs: Optional[Sequence[torch.Tensor]] = None
                                    ) -> List[torch.Tensor]:
    """The insert + conv of up to four streams of one layer in one launch.

    Stream s has x ``xs[s]`` [T, H*ws[s]], weight ``weights[s]`` [H*ws[s], W]
    and cache columns [off_s[s], off_s[s] + ws[s]) of every head.
    ``activation`` and ``use_residual`` are one value for all streams or a
    sequence with one per stream.  Rows find their request either from
    ``seq_idx`` / ``query_start`` or, inside the launch, from
    ``query_start_loc`` with ``num_reqs``.  Returns the outputs.
    """
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    args = _streams_args(xs, weights, cache, positions, block_table, slot_mapping, off_s, ws,
                         block_size, activation, use_residual, seq_idx, query_start,
                         query_start_loc, num_reqs, outs)
    if args is None:
        return list(outs)
    rc = _lib.load().sconv_fused_insert_conv_streams(*args, _stream(xs[0]))
    _lib.check(rc, "sconv_fused_insert_conv_streams")
    return list(outs)


def sconv_fused_plan(xs: Sequence[torch.Tensor], weights: Sequence[torch.Tensor],
                     cache: torch.Tensor, positions: torch.Tensor, block_table: torch.Tensor,
                     slot_mapping: torch.Tensor, off_s: Sequence[int], ws: Sequence[int],
                     block_size: int, activation=None, use_residual=True,
                     seq_idx: Optional[torch.Tensor] = None,
                     query_start: Optional[torch.Tensor] = None,
                     query_start_loc: Optional[torch.Tensor] = None,
                     num_reqs: Optional[int] = None,
                     outs: Optional[Sequence[torch.Tensor]] = None,
                     gather: Optional[tuple] = None) -> dict:
    """The launch sconv_fused_insert_conv_streams (or, with ``gather`` =
    (src, abs_positions, real_count_gpu, out, d_conv),
    sconv_fused_insert_conv_gather) would make for these arguments, as a
    dict of the plan's fields; nothing is launched."""
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    plan = _lib.FusedPlan()
    args = _streams_args(xs, weights, cache, positions, block_table, slot_mapping, off_s, ws,
                         block_size, activation, use_residual, seq_idx, query_start,
                         query_start_loc, num_reqs, outs)
    g = None if gather is None else _window_gather(*gather)[0]
    if args is not None:
        rc = _lib.load().sconv_fused_plan(*args, None if g is None else ctypes.byref(g),
                                          ctypes.byref(plan))
        _lib.check(rc, "sconv_fused_plan")
    return {name: getattr(plan, name) for name, _ in _lib.FusedPlan._fields_}


def _streams_args(xs, weights, cache, positions, block_table, slot_mapping, off_s, ws,
                  block_size, activation, use_residual, seq_idx, query_start, query_start_loc,
                  num_reqs, outs):
    """Checked C arguments of the multi-stream entry points (without the
    stream), or None when there is nothing to launch."""
    n = len(xs)
    if not (len(weights) == len(off_s) == len(ws) == n):
        raise ValueError("xs, weights, off_s and ws need one entry per stream")
    acts = list(activation) if isinstance(activation, (list, tuple)) else [activation] * n
    ress = list(use_residual) if isinstance(use_residual, (list, tuple)) else [use_residual] * n
    if len(acts) != n or len(ress) != n or len(outs) != n:
        raise ValueError("activation, use_residual and outs need one entry per stream")
    T = xs[0].shape[0] if n else 0
    if n == 0 or T == 0:
        return None
    if any(x.shape[0] != T for x in xs):
        raise ValueError("every stream needs the same rows T")
    dt = None
    for x, w, o, a, b in zip(xs, weights, outs, off_s, ws):
        dt = _fused_checks(x, w, cache, positions, block_table, slot_mapping, a, b, block_size, o)
    if any(w.shape[1] != weights[0].shape[1] for w in weights):
        raise ValueError("every stream needs the same filter width W")
    if any(x.dtype != xs[0].dtype for x in xs):
        raise TypeError("every stream needs the same element type")
    if query_start_loc is not None:
        if seq_idx is not None or query_start is not None or num_reqs is None:
            raise ValueError("give query_start_loc with num_reqs, or seq_idx and query_start")
        _dev(query_start_loc)
        _vec(query_start_loc, torch.int32, "query_start_loc", num_reqs + 1)
        _table_rows(block_table, num_reqs)
    else:
        if seq_idx is None or query_start is None:
            raise ValueError("give query_start_loc with num_reqs, or seq_idx and query_start")
        _dev(seq_idx, query_start)
        _vec(seq_idx, torch.int32, "seq_idx", T)
        _vec(query_start, torch.int32, "query_start", T)
    arr = (_lib.StreamT * n)()
    for i, (x, w, o) in enumerate(zip(xs, weights, outs)):
        arr[i] = _lib.StreamT(_ptr(x), x.stride(0), _ptr(w), w.stride(0), w.stride(1), _ptr(o),
                              o.stride(0), int(off_s[i]), int(ws[i]), _act(acts[i]),
                              int(bool(ress[i])))
    nb, H, N, D = cache.shape
    return (arr, n, _ptr(cache), nb, H, N, D, cache.stride(0), cache.stride(1), cache.stride(2),
            _ptr(positions), _ptr(block_table), block_table.stride(0), block_table.shape[1],
            _ptr(seq_idx), _ptr(query_start), _ptr(query_start_loc),
            int(num_reqs) if num_reqs is not None else 0, _ptr(slot_mapping), T,
            weights[0].shape[1], dt)


def causal_conv1d_varlen_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                             conv_states: torch.Tensor, query_start_loc: torch.Tensor,
                             cache_indices: Optional[torch.Tensor],
                             has_initial_state: Optional[torch.Tensor], silu_activation: bool,
                             pad_slot_id: int = -1, out: Optional[torch.Tensor] = None
                             ) -> torch.Tensor:
    """Varlen causal conv1d over channel-major x [dim, total_T].

    conv_states [num_slots, dim, W-1] is updated in place.  With ``out`` None
    the result overwrites x (in place, as the source op does) and x is
    returned.
    """
    if out is None:
        out = x
    if x.dim() != 2 or weight.dim() != 2 or conv_states.dim() != 3:
        raise ValueError("x [dim, total_T], weight [dim, W], conv_states [slots, dim, W-1]")
    dim, total_T = x.shape
    W = weight.shape[1]
    batch = query_start_loc.numel() - 1
    _dev(x, weight, bias, conv_states, query_start_loc, cache_indices, has_initial_state, out)
    dt = _dtype(x)
    for t in (weight, conv_states, out) + ((bias,) if bias is not None else ()):
        if t.dtype != x.dtype:
            raise TypeError("x, weight, bias, conv_states and out must share one element type")
    if weight.shape[0] != dim or conv_states.shape[1] != dim or conv_states.shape[2] != W - 1:
        raise ValueError("weight / conv_states shapes do not match x")
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    if bias is not None:
        _vec(bias, x.dtype, "bias", dim)
    _vec(query_start_loc, torch.int32, "query_start_loc")
    if cache_indices is not None:
        _vec(cache_indices, torch.int32, "cache_indices", batch)
    hi = None
    if has_initial_state is not None:
        hi = has_initial_state
        if hi.dtype == torch.bool:
            hi = hi.view(torch.uint8)
        _vec(hi, torch.uint8, "has_initial_state", batch)
    rc = _lib.load().causal_conv1d_varlen_fwd(
        _ptr(x), x.stride(0), x.stride(1), _ptr(weight), weight.stride(0), weight.stride(1),
        _ptr(bias), _ptr(conv_states), conv_states.shape[0], conv_states.stride(0),
        conv_states.stride(1), conv_states.stride(2), _ptr(query_start_loc), batch,
        _ptr(cache_indices), _ptr(hi), _ptr(out), out.stride(0), out.stride(1), dim, total_T,
        W, dt, _lib.ACT_SILU if silu_activation else _lib.ACT_NONE, int(pad_slot_id), _stream(x))
    _lib.check(rc, "causal_conv1d_varlen_fwd")
    return out


def causal_conv1d_update(x: torch.Tensor, conv_state: torch.Tensor, weight: torch.Tensor,
                         bias: Optional[torch.Tensor], silu_activation: bool,
                         cache_seqlens: Optional[torch.Tensor] = None,
                         conv_state_indices: Optional[torch.Tensor] = None,
                         pad_slot_id: int = -1, out: Optional[torch.Tensor] = None
                         ) -> torch.Tensor:
    """One decode step: x [batch, dim]; conv_state [num_slots, dim, W-1]
    updated in place.  With ``out`` None the result overwrites x."""
    if out is None:
        out = x
    if x.dim() != 2 or weight.dim() != 2 or conv_state.dim() != 3:
        raise ValueError("x [batch, dim], weight [dim, W], conv_state [slots, dim, W-1]")
    batch, dim = x.shape
    W = weight.shape[1]
    _dev(x, conv_state, weight, bias, conv_state_indices, out)
    dt = _dtype(x)
    for t in (weight, conv_state, out) + ((bias,) if bias is not None else ()):
        if t.dtype != x.dtype:
            raise TypeError("x, weight, bias, conv_state and out must share one element type")
    if x.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("x and out need contiguous channels")
    if weight.shape[0] != dim or conv_state.shape[1] != dim or conv_state.shape[2] != W - 1:
        raise ValueError("weight / conv_state shapes do not match x")
    if bias is not None:
        _vec(bias, x.dtype, "bias", dim)
    if conv_state_indices is not None:
        _vec(conv_state_indices, torch.int32, "conv_state_indices", batch)
    if cache_seqlens is not None:
        _dev(cache_seqlens)
        _vec(cache_seqlens, torch.int32, "cache_seqlens", batch)
    rc = _lib.load().causal_conv1d_update(
        _ptr(x), x.stride(0), _ptr(conv_state), conv_state.shape[0], conv_state.stride(0),
        conv_state.stride(1), conv_state.stride(2), _ptr(weight), weight.stride(0),
        weight.stride(1), _ptr(bias), _ptr(cache_seqlens), _ptr(conv_state_indices), _ptr(out),
        out.stride(0), batch, dim, W, dt, _lib.ACT_SILU if silu_activation else _lib.ACT_NONE,
        int(pad_slot_id), _stream(x))
    _lib.check(rc, "causal_conv1d_update")
    return out


def causal_conv1d_update_tokens(x: torch.Tensor, conv_state: torch.Tensor, weight: torch.Tensor,
                                bias: Optional[torch.Tensor], silu_activation: bool,
                                cache_seqlens: Optional[torch.Tensor] = None,
                                conv_state_indices: Optional[torch.Tensor] = None,
                                pad_slot_id: int = -1, out: Optional[torch.Tensor] = None
                                ) -> torch.Tensor:
    """seqlen decode tokens per row: x [batch, dim, seqlen] (any strides);
    conv_state [num_slots, dim, state_len] (W-1 <= state_len <= 8) updated in
    place, a ring indexed by position when ``cache_seqlens`` (int32 [batch])
    is given.  With ``out`` None the result overwrites x."""
    if out is None:
        out = x
    if x.dim() != 3 or weight.dim() != 2 or conv_state.dim() != 3 or out.shape != x.shape:
        raise ValueError("x and out [batch, dim, seqlen], weight [dim, W], "
                         "conv_state [slots, dim, state_len]")
    batch, dim, seqlen = x.shape
    W = weight.shape[1]
    _dev(x, conv_state, weight, bias, conv_state_indices, cache_seqlens, out)
    dt = _dtype(x)
    for t in (weight, conv_state, out) + ((bias,) if bias is not None else ()):
        if t.dtype != x.dtype:
            raise TypeError("x, weight, bias, conv_state and out must share one element type")
    if weight.shape[0] != dim or conv_state.shape[1] != dim:
        raise ValueError("weight / conv_state shapes do not match x")
    if bias is not None:
        _vec(bias, x.dtype, "bias", dim)
    if conv_state_indices is not None:
        _vec(conv_state_indices, torch.int32, "conv_state_indices", batch)
    if cache_seqlens is not None:
        _vec(cache_seqlens, torch.int32, "cache_seqlens", batch)
    rc = _lib.load().causal_conv1d_update_tokens(
        _ptr(x), x.stride(0), x.stride(1), x.stride(2), seqlen, _ptr(conv_state),
        conv_state.shape[0], conv_state.shape[2], conv_state.stride(0), conv_state.stride(1),
        conv_state.stride(2), _ptr(weight), weight.stride(0), weight.stride(1), _ptr(bias),
        _ptr(cache_seqlens), _ptr(conv_state_indices), _ptr(out), out.stride(0), out.stride(1),
        out.stride(2), batch, dim, W, dt, _lib.ACT_SILU if silu_activation else _lib.ACT_NONE,
        int(pad_slot_id), _stream(x))
    _lib.check(rc, "causal_conv1d_update_tokens")
    return out


def gather_intermediate_conv_window(src: torch.Tensor, abs_positions: torch.Tensor,
                                    real_count_gpu: torch.Tensor, out: torch.Tensor,
                                    d_conv: int) -> None:
    """Gather length-d_conv windows of src[0] ending before abs_positions
    into out [max_count, conv_dim, d_conv] for the first real_count slots
    (count read on the device)."""
    g, dt = _window_gather(src, abs_positions, real_count_gpu, out, d_conv)
    rc = _lib.load().gather_intermediate_conv_window(
        g.src, g.seq_len, g.conv_dim, g.src_stride_s, g.src_stride_c, g.abs_positions,
        g.real_count, g.max_count, g.out, g.out_slot_stride, g.d_conv, dt, _stream(src))
    _lib.check(rc, "gather_intermediate_conv_window")


def _window_gather(src, abs_positions, real_count_gpu, out, d_conv):
    """Checked sconv_window_gather_t of a window gather, and its dtype code."""
    if src.dim() != 3 or out.dim() != 3:
        raise ValueError("src [batch, seq_len, conv_dim], out [max_count, conv_dim, d_conv]")
    _dev(src, abs_positions, real_count_gpu, out)
    dt = _dtype(src)
    if out.dtype != src.dtype:
        raise TypeError("src and out must share one element type")
    max_count, conv_dim, dc = out.shape
    if dc != d_conv or conv_dim != src.shape[2]:
        raise ValueError("out must be [max_count, conv_dim, d_conv]")
    if out.stride(2) != 1 or out.stride(1) != d_conv:
        raise ValueError("out slots must be dense (conv_dim, d_conv)")
    _vec(abs_positions, torch.int32, "abs_positions", max_count)
    _vec(real_count_gpu, torch.int32, "real_count_gpu", 1)
    g = _lib.WindowGather(_ptr(src), src.shape[1], conv_dim, src.stride(1), src.stride(2),
                          _ptr(abs_positions), _ptr(real_count_gpu), max_count, _ptr(out),
                          out.stride(0), d_conv)
    return g, dt


def sconv_fused_insert_conv_gather(xs: Sequence[torch.Tensor], weights: Sequence[torch.Tensor],
                                   cache: torch.Tensor, positions: torch.Tensor,
                                   block_table: torch.Tensor, slot_mapping: torch.Tensor,
                                   off_s: Sequence[int], ws: Sequence[int], block_size: int,
                                   gather_src: torch.Tensor, abs_positions: torch.Tensor,
                                   real_count_gpu: torch.Tensor, gather_out: torch.Tensor,
                                   d_conv: int, activation=None, use_residual=True,
                                   seq_idx: Optional[torch.Tensor] = None,
                                   query_start: Optional[torch.Tensor] = None,
                                   query_start_loc: Optional[torch.Tensor] = None,
                                   num_reqs: Optional[int] = None,
                                   outs: Optional[Sequence[torch.Tensor]] = None
                                   ) -> List[torch.Tensor]:
    """sconv_fused_insert_conv_streams and gather_intermediate_conv_window
    (gather_src, abs_positions, real_count_gpu, gather_out, d_conv) in one
    launch.  Returns the conv outputs; gather_out is written in place."""
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    g, gdt = _window_gather(gather_src, abs_positions, real_count_gpu, gather_out, d_conv)
    args = _streams_args(xs, weights, cache, positions, block_table, slot_mapping, off_s, ws,
                         block_size, activation, use_residual, seq_idx, query_start,
                         query_start_loc, num_reqs, outs)
    if args is None:  # no rows: the gather alone
        gather_intermediate_conv_window(gather_src, abs_positions, real_count_gpu, gather_out,
                                        d_conv)
        return list(outs)
    if gdt != args[-1]:
        raise TypeError("the gather and the conv must share one element type")
    rc = _lib.load().sconv_fused_insert_conv_gather(*args, ctypes.byref(g), _stream(xs[0]))
    _lib.check(rc, "sconv_fused_insert_conv_gather")
    return list(outs)


def gather_intermediate_ssm_state(states: torch.Tensor, chunk_indices: torch.Tensor,
                                  real_count_gpu: torch.Tensor, out: torch.Tensor) -> None:
    """Copy states[chunk_indices[i]] into out[i] for the first real_count
    slots (count read on the device).  states [num_chunks, *state_shape],
    out [max_count, *state_shape]; each row must be dense."""
    _dev(states, chunk_indices, real_count_gpu, out)
    dt = _dtype(states)
    if out.dtype != states.dtype:
        raise TypeError("states and out must share one element type")
    if states.shape[1:] != out.shape[1:]:
        raise ValueError("states and out rows must have one shape")
    flat = 1
    for d in states.shape[1:]:
        flat *= d
    for t, name in ((states, "states"), (out, "out")):
        if t.dim() > 1 and not t[0].is_contiguous():
            raise ValueError(f"{name} rows must be dense")
    max_count = out.shape[0]
    _vec(chunk_indices, torch.int64, "chunk_indices", max_count)
    _vec(real_count_gpu, torch.int32, "real_count_gpu", 1)
    rc = _lib.load().gather_intermediate_ssm_state(
        _ptr(states), states.shape[0], flat, states.stride(0) if states.dim() > 1 else 1,
        _ptr(chunk_indices), _ptr(real_count_gpu), max_count, _ptr(out),
        out.stride(0) if out.dim() > 1 else 1, dt, _stream(states))
    _lib.check(rc, "gather_intermediate_ssm_state")
