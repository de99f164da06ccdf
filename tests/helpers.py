"""Shared test plumbing: tensor <-> numpy marshalling and comparisons.

Nothing here computes the convolution; it only moves data between the
generators, the oracle and the GPU library, and compares results.
"""
from __future__ import annotations

import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor; bfloat16 becomes its uint16 bit pattern."""
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def from_np(a: np.ndarray, like: torch.dtype) -> torch.Tensor:
    if like == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def as_float(a: np.ndarray) -> np.ndarray:
    """Values of a float32/float64/bf16-bits array as float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def bits(a: np.ndarray) -> np.ndarray:
    """Bit patterns, so that NaN == NaN in exactness checks."""
    if a.dtype == np.uint16:
        return a
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float64:
        return a.view(np.uint64)
    return a


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str = ""):
    a, b = bits(np.ascontiguousarray(a)), bits(np.ascontiguousarray(b))
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = np.nonzero(a != b)
    if bad[0].size:
        idx = tuple(int(i[0]) for i in bad)
        raise AssertionError(f"{what}: {bad[0].size} elements differ; first at {idx}: "
                             f"{a[idx]:#x} vs {b[idx]:#x}")


# Tolerances for floating outputs (GPU: fp32 accumulate, any tap order).
TOL = {
    "f32": dict(rtol=1e-5, atol=1e-6),
    "bf16": dict(rtol=1.6e-2, atol=1e-2),
}


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", mask=None):
    """Every compared value finite on both sides and within the dtype's
    tolerance.  Live outputs come from finite inputs, so a NaN or an
    infinity on either side is a failure: the generators fill every cache
    and state position an op must not read with NaN, and a stray read must
    not pass by showing up on both sides."""
    g, r = as_float(got), as_float(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    tol = TOL[dtype]
    assert g.shape == r.shape, (what, g.shape, r.shape)
    for side, v in (("got", g), ("reference", r)):
        nf = ~np.isfinite(v)
        if nf.any():
            i = np.flatnonzero(nf)[0]
            raise AssertionError(f"{what}: {int(nf.sum())}/{v.size} non-finite values in the "
                                 f"{side} side; first flat index {i}: {v.flat[i]!r}")
    err = np.abs(g - r)
    lim = tol["atol"] + tol["rtol"] * np.abs(r)
    bad = ~(err <= lim)
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside atol={tol['atol']} rtol={tol['rtol']}; "
            f"first flat index {i}: got {g.flat[i]!r} want {r.flat[i]!r}")


def assert_finite(a: np.ndarray, what: str = ""):
    """Values (float32/float64 or bf16 bits) are all finite."""
    v = as_float(np.asarray(a)) if np.asarray(a).dtype != np.float64 else np.asarray(a)
    nf = ~np.isfinite(v)
    if nf.any():
        i = np.flatnonzero(nf)[0]
        raise AssertionError(f"{what}: {int(nf.sum())}/{v.size} non-finite values; first flat "
                             f"index {i}: {v.flat[i]!r}")
