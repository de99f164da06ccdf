"""ctypes loader for libsconv.so (the HIP library built from csrc/).

torch is imported first so that the process has exactly one HIP runtime:
libsconv.so links ``libamdhip64.so.7`` by soname, which then resolves to the
runtime torch already loaded.  There is no fallback: if the library is not
built, importing the binding fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime this library binds to)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsconv.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
F32, BF16 = 0, 1
ACT_NONE, ACT_SILU = 0, 1

EXPORTS = (
    "sconv_last_error",
    "sconv_version",
    "sconv_init",
    "sconv_seq_metadata",
    "sconv_fused_insert_conv",
    "sconv_fused_insert_conv_qsl",
    "sconv_fused_insert_conv_streams",
    "sconv_fused_plan",
    "sconv_fused_insert_conv_gather",
    "causal_conv1d_varlen_fwd",
    "causal_conv1d_update",
    "causal_conv1d_update_tokens",
    "gather_intermediate_conv_window",
    "gather_intermediate_ssm_state",
)

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64


class StreamT(ctypes.Structure):
    """sconv_stream_t of include/sconv.h (one conv stream of a layer)."""
    _fields_ = [("x", P), ("x_row_stride", I64), ("weight", P), ("w_stride_c", I64),
                ("w_stride_k", I64), ("out", P), ("out_row_stride", I64), ("off_s", I32),
                ("ws", I32), ("activation", I32), ("use_residual", I32)]


class FusedPlan(ctypes.Structure):
    """sconv_fused_plan_t of include/sconv.h (the launch a fused call makes)."""
    _fields_ = [("lane_elems", I32), ("rows_per_tile", I32), ("request_mode", I32),
                ("rows_per_request", I32), ("bt_row_entries", I32), ("stream_x_loads", I32),
                ("stream_hist_loads", I32), ("tile_major", I32), ("wg_threads", I32),
                ("gather_mode", I32), ("waves", I64), ("workgroups", I64),
                ("early_inserts", I32)]


class WindowGather(ctypes.Structure):
    """sconv_window_gather_t of include/sconv.h (a conditional window gather)."""
    _fields_ = [("src", P), ("seq_len", I64), ("conv_dim", I32), ("src_stride_s", I64),
                ("src_stride_c", I64), ("abs_positions", P), ("real_count", P),
                ("max_count", I32), ("out", P), ("out_slot_stride", I64), ("d_conv", I32)]


_SIGS = {
    "sconv_init": [],
    "sconv_seq_metadata": [P, I32, I64, I64, P, I64, P, I64, P],
    "sconv_fused_insert_conv": [P, I64, P, I64, I64, P, I64, I32, I32, I32, I64, I64, I64,
                                P, P, I64, I32, P, P, P, P, I64, I64, I32, I32, I32, I32,
                                I32, I32, P],
    "sconv_fused_insert_conv_qsl": [P, I64, P, I64, I64, P, I64, I32, I32, I32, I64, I64, I64,
                                    P, P, I64, I32, P, I32, P, P, I64, I64, I32, I32, I32,
                                    I32, I32, I32, P],
    "sconv_fused_insert_conv_streams": [ctypes.POINTER(StreamT), I32, P, I64, I32, I32, I32,
                                        I64, I64, I64, P, P, I64, I32, P, P, P, I32, P, I64,
                                        I32, I32, P],
    "sconv_fused_plan": [ctypes.POINTER(StreamT), I32, P, I64, I32, I32, I32, I64, I64, I64,
                         P, P, I64, I32, P, P, P, I32, P, I64, I32, I32,
                         ctypes.POINTER(WindowGather), ctypes.POINTER(FusedPlan)],
    "sconv_fused_insert_conv_gather": [ctypes.POINTER(StreamT), I32, P, I64, I32, I32, I32, I64,
                                       I64, I64, P, P, I64, I32, P, P, P, I32, P, I64, I32, I32,
                                       ctypes.POINTER(WindowGather), P],
    "causal_conv1d_varlen_fwd": [P, I64, I64, P, I64, I64, P, P, I64, I64, I64, I64, P, I32,
                                 P, P, P, I64, I64, I32, I64, I32, I32, I32, I32, P],
    "causal_conv1d_update": [P, I64, P, I64, I64, I64, I64, P, I64, I64, P, P, P, P, I64,
                             I32, I32, I32, I32, I32, I32, P],
    "causal_conv1d_update_tokens": [P, I64, I64, I64, I32, P, I64, I32, I64, I64, I64, P, I64,
                                    I64, P, P, P, P, I64, I64, I64, I32, I32, I32, I32, I32,
                                    I32, P],
    "gather_intermediate_conv_window": [P, I64, I32, I64, I64, P, P, I32, P, I64, I32, I32, P],
    "gather_intermediate_ssm_state": [P, I64, I64, I64, P, P, I32, P, I64, I32, P],
}


class LibsconvError(RuntimeError):
    pass


_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (built beforehand by ``depthwise_causal_conv1d_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m depthwise_causal_conv1d_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.sconv_last_error.restype = ctypes.c_char_p
        lib.sconv_last_error.argtypes = []
        lib.sconv_version.restype = ctypes.c_char_p
        lib.sconv_version.argtypes = []
        for name, args in _SIGS.items():
            try:
                fn = getattr(lib, name)
            except AttributeError:
                raise ImportError(
                    f"{LIB_PATH} lacks {name}: it is older than the sources; rebuild it with "
                    "`python -m depthwise_causal_conv1d_amd.build`") from None
            fn.restype = ctypes.c_int
            fn.argtypes = args
        _lib = lib
    return _lib


def check(rc: int, what: str):
    if rc == OK:
        return
    msg = load().sconv_last_error().decode()
    if rc == ERR_INVALID:
        raise ValueError(msg or f"{what}: invalid argument")
    if rc == ERR_UNSUPPORTED:
        raise NotImplementedError(msg or f"{what}: unsupported")
    raise LibsconvError(msg or f"{what}: HIP error")
