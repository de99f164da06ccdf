"""Plain CPU oracle for the paged depthwise causal short convolution.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers; the product package
never imports this module, and this module imports nothing from it.

The arithmetic lives in ``sconv_oracle.c`` (plain C, double precision, one
rounding to the output type).  This file only marshals numpy arrays into it.
Arrays hold float32, float64 or bfloat16 *bit patterns* (numpy ``uint16``);
the element type of a call is taken from ``x``.

Every function cites the page passage it follows in ``sconv_oracle.c``;
``fused_insert_conv_streams`` is the single-stream op applied per stream.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sconv_oracle.c")
# SCONV_ORACLE_LIB names another build of sconv_oracle.c to load instead
# (the mutation tests plant mistakes in copies of the source); build() then
# leaves it as it is.
_OVERRIDE = os.environ.get("SCONV_ORACLE_LIB")
_LIB_PATH = _OVERRIDE or os.path.join(_HERE, "libsconv_oracle.so")

F32, BF16, F64 = 0, 1, 2
ACT_NONE, ACT_SILU = 0, 1

_ERRORS = {
    -1: "bad scalar argument",
    -2: "seq_idx outside [0, num_reqs)",
    -3: "logical block outside [0, max_blocks)",
    -4: "physical block outside [0, num_blocks)",
    -5: "x row outside [0, T)",
    -6: "state slot outside [0, num_slots)",
    -7: "state row outside [0, num_chunks)",
}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    if _OVERRIDE:
        return _LIB_PATH
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(compile_command(_SRC, tmp))
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def compile_command(src: str, out: str):
    """The gcc command that builds the oracle library from `src`."""
    return ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-pthread",
            "-o", out, src, "-lm"]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.oracle_round_bf16.restype = ctypes.c_uint16
        _lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        _lib.oracle_bf16_to_double.restype = ctypes.c_double
        _lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        _lib.oracle_silu.restype = ctypes.c_double
        _lib.oracle_silu.argtypes = [ctypes.c_double]
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle element type must be float32, float64 or uint16 (bf16 bits), got {a.dtype}")


def _p(a):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


def _es(a: np.ndarray, axis: int) -> int:
    return a.strides[axis] // a.itemsize


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _act(activation) -> int:
    if activation in (None, "none", False, ACT_NONE):
        return ACT_NONE
    if activation in ("silu", "swish", True, ACT_SILU):
        return ACT_SILU
    raise ValueError(f"unknown activation {activation!r}")


I64 = ctypes.c_int64
I32 = ctypes.c_int32


# ---------------------------------------------------------------- scalars

def round_bf16(v: float) -> int:
    """bfloat16 bit pattern nearest to ``v`` (ties to even)."""
    return int(_load().oracle_round_bf16(float(v)))


def bf16_to_float(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits)))


def silu(v: float) -> float:
    return float(_load().oracle_silu(float(v)))


# ---------------------------------------------------------------- ops

def seq_metadata(query_start_loc, num_reqs: int, num_actual: int, num_padded: int | None = None):
    """Returns (seq_idx, query_start) int32 arrays of length num_padded."""
    lib = _load()
    if num_padded is None:
        num_padded = num_actual
    qsl = _c(query_start_loc, np.int32)
    seq_idx = np.full(num_padded, -7, np.int32)
    qs = np.full(num_padded, -7, np.int32)
    rc = lib.oracle_seq_metadata(_p(qsl), I32(num_reqs), I64(num_actual), I64(num_padded),
                                 _p(seq_idx), _p(qs))
    _check(rc, "seq_metadata")
    return seq_idx, qs


def fused_insert_conv(x, weight, cache, positions, block_table, seq_idx, slot_mapping,
                      query_start, off_s: int, ws: int, block_size: int,
                      activation=None, use_residual: bool = True, out_init=None,
                      threads: int = 1):
    """Returns (out, cache_after).  ``cache`` itself is not modified.

    x [T, H*ws], weight [H*ws, W], cache [num_blocks, H, N, D],
    positions int64 [T], block_table int32 [num_reqs, max_blocks],
    seq_idx / query_start int32 [T], slot_mapping int64 [T].
    ``out_init`` (default zeros) supplies the values PAD rows keep.
    ``threads`` > 1 splits the rows over that many host threads (same bits).
    """
    lib = _load()
    x = _c(x)
    dt = _dtype_code(x)
    w = _c(weight, x.dtype)
    cache_in = _c(cache, x.dtype)
    cache_out = cache_in.copy()
    T = x.shape[0]
    nb, H, N, D = cache_in.shape
    if N != block_size:
        raise ValueError("cache block dim != block_size")
    bt = _c(block_table, np.int32)
    if bt.ndim != 2:
        raise ValueError("block_table must be 2-D")
    out = np.zeros_like(x) if out_init is None else np.array(out_init, dtype=x.dtype, copy=True)
    # Keep every marshalled array bound to a name until the call returns.
    pos = _c(positions, np.int64)
    si = _c(seq_idx, np.int32)
    sm = _c(slot_mapping, np.int64)
    qs = _c(query_start, np.int32)
    if not (pos.shape[0] >= T and si.shape[0] >= T and sm.shape[0] >= T and qs.shape[0] >= T):
        raise ValueError("per-token arrays shorter than T")
    args = (_p(x), I64(_es(x, 0)), _p(w), I64(_es(w, 0)), I64(_es(w, 1)),
            _p(cache_in), _p(cache_out), I64(nb), I32(H), I32(N), I32(D),
            I64(_es(cache_in, 0)), I64(_es(cache_in, 1)), I64(_es(cache_in, 2)),
            _p(pos), _p(bt), I64(_es(bt, 0)), I32(bt.shape[0]), I32(bt.shape[1]),
            _p(si), _p(sm), _p(qs),
            _p(out), I64(_es(out, 0)), I64(T), I32(off_s), I32(ws), I32(w.shape[1]),
            dt, _act(activation), int(bool(use_residual)))
    if threads > 1:
        rc = lib.oracle_fused_insert_conv_mt(*args, I32(threads))
    else:
        rc = lib.oracle_fused_insert_conv(*args)
    _check(rc, "fused_insert_conv")
    return out, cache_out


def fused_insert_conv_streams(streams, cache, positions, block_table, seq_idx, slot_mapping,
                              query_start, block_size: int):
    """Insert + conv of several conv streams of one layer (vLLM sconv page,
    module description: a layer's streams share one paged cache, each in its
    own column sub-range of every head).  By definition this is the
    single-stream op applied to each stream in turn, the cache carried from
    one to the next.

    ``streams``: one dict per stream with x, weight, off_s, ws, activation,
    use_residual and optionally out_init.  Returns ([out per stream],
    cache_after); ``cache`` itself is not modified.
    """
    outs = []
    c = cache
    for st in streams:
        o, c = fused_insert_conv(st["x"], st["weight"], c, positions, block_table, seq_idx,
                                 slot_mapping, query_start, st["off_s"], st["ws"], block_size,
                                 st.get("activation"), st.get("use_residual", True),
                                 out_init=st.get("out_init"))
        outs.append(o)
    return outs, c


def causal_conv1d_varlen_fwd(x, weight, bias, conv_states, query_start_loc, cache_indices,
                             has_initial_state, activation, pad_slot_id: int = -1,
                             out_init=None, threads: int = 1):
    """Returns (out, conv_states_after).  ``threads`` > 1 splits the
    channels over that many host threads (same bits).

    x [dim, total_T] (channel-major), weight [dim, W], bias [dim] or None,
    conv_states [num_slots, dim, W-1], query_start_loc int32 [batch+1],
    cache_indices int32 [batch] or None, has_initial_state bool [batch] or None.
    """
    lib = _load()
    x = _c(x)
    dt = _dtype_code(x)
    w = _c(weight, x.dtype)
    b = _c(bias, x.dtype)
    st_in = _c(conv_states, x.dtype)
    st_out = st_in.copy()
    qsl = _c(query_start_loc, np.int32)
    batch = qsl.shape[0] - 1
    ci = _c(cache_indices, np.int32)
    hi = None if has_initial_state is None else _c(np.asarray(has_initial_state).astype(np.uint8))
    dim, total_T = x.shape
    out = np.zeros_like(x) if out_init is None else np.array(out_init, dtype=x.dtype, copy=True)
    args = (_p(x), I64(_es(x, 0)), I64(_es(x, 1)), _p(w), I64(_es(w, 0)), I64(_es(w, 1)), _p(b),
            _p(st_in), _p(st_out), I64(st_in.shape[0]),
            I64(_es(st_in, 0)), I64(_es(st_in, 1)), I64(_es(st_in, 2)),
            _p(qsl), I32(batch), _p(ci), _p(hi), _p(out), I64(_es(out, 0)), I64(_es(out, 1)),
            I32(dim), I64(total_T), I32(w.shape[1]), dt, _act(activation), I32(pad_slot_id))
    if threads > 1:
        rc = lib.oracle_causal_conv1d_varlen_fwd_mt(*args, I32(threads))
    else:
        rc = lib.oracle_causal_conv1d_varlen_fwd(*args)
    _check(rc, "causal_conv1d_varlen_fwd")
    return out, st_out


def causal_conv1d_update(x, conv_states, weight, bias, activation, conv_state_indices=None,
                         pad_slot_id: int = -1, out_init=None):
    """Returns (out, conv_states_after).  x [batch, dim]."""
    lib = _load()
    x = _c(x)
    dt = _dtype_code(x)
    w = _c(weight, x.dtype)
    b = _c(bias, x.dtype)
    st_in = _c(conv_states, x.dtype)
    st_out = st_in.copy()
    ci = _c(conv_state_indices, np.int32)
    batch, dim = x.shape
    out = np.zeros_like(x) if out_init is None else np.array(out_init, dtype=x.dtype, copy=True)
    rc = lib.oracle_causal_conv1d_update(
        _p(x), I64(_es(x, 0)), _p(st_in), _p(st_out), I64(st_in.shape[0]),
        I64(_es(st_in, 0)), I64(_es(st_in, 1)), I64(_es(st_in, 2)),
        _p(w), I64(_es(w, 0)), I64(_es(w, 1)), _p(b), _p(ci), _p(out), I64(_es(out, 0)),
        I32(batch), I32(dim), I32(w.shape[1]), dt, _act(activation), I32(pad_slot_id))
    _check(rc, "causal_conv1d_update")
    return out, st_out


def causal_conv1d_update_tokens(x, conv_states, weight, bias, activation, cache_seqlens=None,
                                conv_state_indices=None, pad_slot_id: int = -1, out_init=None):
    """Returns (out, conv_states_after).  x [batch, dim, seqlen];
    conv_states [num_slots, dim, state_len]; cache_seqlens int32 [batch] or
    None (see oracle_causal_conv1d_update_tokens for both state readings)."""
    lib = _load()
    x = _c(x)
    dt = _dtype_code(x)
    w = _c(weight, x.dtype)
    b = _c(bias, x.dtype)
    st_in = _c(conv_states, x.dtype)
    st_out = st_in.copy()
    cs = _c(cache_seqlens, np.int32)
    ci = _c(conv_state_indices, np.int32)
    batch, dim, seqlen = x.shape
    out = np.zeros_like(x) if out_init is None else np.array(out_init, dtype=x.dtype, copy=True)
    rc = lib.oracle_causal_conv1d_update_tokens(
        _p(x), I64(_es(x, 0)), I64(_es(x, 1)), I64(_es(x, 2)), I32(seqlen), _p(st_in),
        _p(st_out), I64(st_in.shape[0]), I32(st_in.shape[2]), I64(_es(st_in, 0)),
        I64(_es(st_in, 1)), I64(_es(st_in, 2)), _p(w), I64(_es(w, 0)), I64(_es(w, 1)), _p(b),
        _p(cs), _p(ci), _p(out), I64(_es(out, 0)), I64(_es(out, 1)), I64(_es(out, 2)),
        I32(batch), I32(dim), I32(w.shape[1]), dt, _act(activation), I32(pad_slot_id))
    _check(rc, "causal_conv1d_update_tokens")
    return out, st_out


def gather_conv_window(src, abs_positions, real_count: int, out, d_conv: int):
    """Returns a copy of ``out`` with slots < clamp(real_count) filled.

    src [seq_len, conv_dim] (batch row 0), abs_positions int32 [max_count],
    out [max_count, conv_dim, d_conv].
    """
    lib = _load()
    src = np.asarray(src)
    if src.ndim == 3:
        src = src[0]
    src = _c(src)
    dt = _dtype_code(src)
    out = np.array(out, dtype=src.dtype, copy=True, order="C")
    pos = _c(abs_positions, np.int32)
    seq_len, conv_dim = src.shape
    rc = lib.oracle_gather_conv_window(
        _p(src), I64(seq_len), I32(conv_dim), I64(_es(src, 0)), I64(_es(src, 1)), _p(pos),
        I32(real_count), I32(out.shape[0]), _p(out), I64(_es(out, 0)), I32(d_conv), dt)
    _check(rc, "gather_conv_window")
    return out


def gather_ssm_state(states, chunk_indices, real_count: int, out):
    """Returns a copy of ``out`` with slots < clamp(real_count) filled.

    states [num_chunks, *state_shape], chunk_indices int64 [max_count],
    out [max_count, *state_shape] (rows are flattened).
    """
    lib = _load()
    st = _c(states)
    dt = _dtype_code(st)
    num_chunks = st.shape[0]
    st2 = st.reshape(num_chunks, -1)
    out = np.array(out, dtype=st.dtype, copy=True, order="C")
    out2 = out.reshape(out.shape[0], -1)
    if out2.shape[1] != st2.shape[1]:
        raise ValueError("states and out rows differ in size")
    idx = _c(chunk_indices, np.int64)
    rc = lib.oracle_gather_ssm_state(
        _p(st2), I64(num_chunks), I64(st2.shape[1]), I64(_es(st2, 0)), _p(idx), I32(real_count),
        I32(out2.shape[0]), _p(out2), I64(_es(out2, 0)), dt)
    _check(rc, "gather_ssm_state")
    return out
