"""The branch-free division by a host scalar d used by the fused kernel
(block size N, and rows per request k): q = (t + ((v - t) >> s1)) >> s2 with
t = mulhi(v, magic), parameters from the host (d = 1: (0, 0, 0); d = 2^k:
(1, 1, k-1); otherwise the round-up magic number of Granlund & Montgomery).
This transcribes the host parameter routine and the device formula in
uint32 arithmetic and checks them against integer division.  The GPU parity
tests cover the same divisors end to end (N = 1, 4, 8, 16, 24, 32 and
1 000 003; k = 1 and 4)."""
from __future__ import annotations

import numpy as np
import pytest

M32 = (1 << 32) - 1


def magic_for(d: int):
    if d == 1:
        return 0, 0, 0
    if d & (d - 1) == 0:
        return 1, 1, d.bit_length() - 2          # ctz(d) - 1
    l = (d - 1).bit_length()                       # ceil(log2 d)
    return ((1 << 32) * ((1 << l) - d)) // d + 1, 1, l - 1


def div_magic(v: np.ndarray, magic: int, s1: int, s2: int) -> np.ndarray:
    v = v.astype(np.uint64)
    t = (v * np.uint64(magic)) >> np.uint64(32)    # mulhi of two uint32
    return (t + (((v - t) & np.uint64(M32)) >> np.uint64(s1))) >> np.uint64(s2)


DIVISORS = list(range(1, 65)) + [96, 100, 127, 255, 257, 1000, 4096, 65537, 1_000_003,
                                 (1 << 31) - 1, 1 << 31]


@pytest.mark.parametrize("d", DIVISORS)
def test_division_matches_integer_division(d):
    magic, s1, s2 = magic_for(d)
    assert 0 <= magic <= M32
    rng = np.random.default_rng(d)
    v = np.concatenate([
        np.arange(1 << 20, dtype=np.uint64),                       # every small value
        (np.arange(0, (1 << 22) // d + 2, dtype=np.uint64) * np.uint64(d))[:, None]
        + np.array([0, 1, d - 1], dtype=np.uint64)[None, :] if d > 1 else np.zeros((1, 1), np.uint64),
        rng.integers(0, 1 << 32, 200_000, dtype=np.uint64),        # across 32 bits
        np.arange(M32 - 4096, M32 + 1, dtype=np.uint64),           # the top of the range
    ], axis=None)
    v = v[v <= M32]
    np.testing.assert_array_equal(div_magic(v, magic, s1, s2), v // np.uint64(d))
