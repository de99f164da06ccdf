"""The benchmark's algorithmic byte counts, checked against counts made by
hand on tiny cases (CPU only).  Every roofline figure divides these bytes
by a measured time, so a miscount would misstate every fraction of peak."""
from __future__ import annotations

import os
import sys
from types import SimpleNamespace

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _case(positions, slots, qsl, W=4, N=4, C=8):
    T = len(positions)
    return SimpleNamespace(
        x=torch.zeros(T, C, dtype=torch.bfloat16), C=C, W=W, block_size=N, T=T,
        positions=torch.tensor(positions, dtype=torch.int64),
        slot_mapping=torch.tensor(slots, dtype=torch.int64),
        query_start_loc=torch.tensor(qsl, dtype=torch.int32), num_reqs=len(qsl) - 1)


# One request of 6 rows at positions 10..15 (a 10-token history), row 2 PAD,
# W = 4, N = 4, C = 8 bf16 channels (16 bytes a row).
ONE = dict(positions=list(range(10, 16)), slots=[40, 41, -1, 43, 44, 45], qsl=[0, 6])


def test_whole_launch_by_hand():
    # Live rows 0, 1, 3, 4, 5.  Input rows read: 0..5 (row 2 is PAD but row 3
    # taps it).  History taps: positions 9, 8, 7 (row 0 needs all three, row 1
    # two of them), in blocks 2, 2, 1: two block-table entries.
    # (6 x rows + 3 taps + 2 x 5 writes) x 16 B + weights 8 x 4 x 2 B
    # + 24 B x 6 rows of metadata + 4 B x 2 entries.
    expect = (6 + 3 + 10) * 16 + 64 + 24 * 6 + 4 * 2
    assert bench.fused_algorithmic_bytes(_case(**ONE)) == expect == 520


def test_row_range_cutting_a_request():
    # Rows 3..5 only: they tap rows 0..2 of the same request as input rows
    # (before the range), and no history.  x rows read: 3, 4, 5 and 0, 1, 2.
    expect = (6 + 0 + 2 * 3) * 16 + 64 + 24 * 3
    assert bench.fused_algorithmic_bytes(_case(**ONE), (3, 6)) == expect == 328


def test_first_rows_of_a_range_with_history():
    # Rows 0..1 only: x rows 0 and 1, history taps 9, 8, 7 as above.
    expect = (2 + 3 + 2 * 2) * 16 + 64 + 24 * 2 + 4 * 2
    assert bench.fused_algorithmic_bytes(_case(**ONE), (0, 2)) == expect


def test_decode_rows():
    # Three one-row requests at positions 0, 1 and 5 (W = 4, N = 4): taps
    # {}, {0}, {4, 3, 2} in blocks {}, {0}, {1, 0}; every row live.
    c = _case(positions=[0, 1, 5], slots=[0, 5, 9], qsl=[0, 1, 2, 3])
    expect = (3 + 4 + 2 * 3) * 16 + 64 + 24 * 3 + 4 * 3
    assert bench.fused_algorithmic_bytes(c) == expect


def test_streams_share_metadata_and_table():
    # Two streams over the same rows: each stream's own bytes, with the
    # per-row metadata and the block-table entries counted once.
    a, b = _case(**ONE), _case(**ONE, C=16)
    one_a = bench.fused_algorithmic_bytes(a)
    one_b = bench.fused_algorithmic_bytes(b)
    shared = 24 * 6 + 4 * 2
    assert bench.fused_streams_algorithmic_bytes([a, b]) == one_a + one_b - shared
