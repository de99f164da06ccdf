"""GPU parity: the HIP library (through its C ABI) against the oracle.

Outputs are compared element by element within the stated tolerance
(fp32: rtol 1e-5 + atol 1e-6; bf16 I/O with fp32 accumulation: atol 1e-2,
rtol 1.6e-2).  Integer metadata, cache contents, states and gathered windows
must match bit for bit; PAD rows and dead slots must keep their sentinel.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import (SENTINEL, dtype_name, gpu_fused, gpu_fused_streams, gpu_plan,
                            live_rows, oracle_fused, oracle_fused_streams, written_cache_values)
from tests.helpers import assert_bits_equal, assert_close, assert_finite, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("oracle_lib")]

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import depthwise_causal_conv1d_amd  # noqa: F401  (fails loudly if not built)


def say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ metadata

@pytest.mark.parametrize("seed,R,max_len,extra_pad", [
    (0, 1, 64, 0), (1, 7, 9, 5), (2, 256, 3, 0), (3, 512, 8, 37), (4, 9000, 2, 11),
    (5, 3, 0, 4)])
def test_seq_metadata_bit_exact(seed, R, max_len, extra_pad):
    import depthwise_causal_conv1d_amd as lib
    import oracle
    say(f"metadata seed={seed} R={R}")
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, R)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    num_actual = int(qsl[-1]) + (2 if seed == 1 else 0)
    num_padded = num_actual + extra_pad
    si_ref, qs_ref = oracle.seq_metadata(qsl, R, num_actual, num_padded)
    n = max(num_padded, 1) + 3
    si = torch.full((n,), -9, dtype=torch.int32, device=DEV)
    qs = torch.full((n,), -9, dtype=torch.int32, device=DEV)
    lib.sconv_seq_metadata(torch.from_numpy(qsl).to(DEV), R, num_actual, si, qs, num_padded)
    si_h, qs_h = to_np(si), to_np(qs)
    np.testing.assert_array_equal(si_h[:num_padded], si_ref)
    np.testing.assert_array_equal(qs_h[:num_padded], qs_ref)
    assert (si_h[num_padded:] == -9).all() and (qs_h[num_padded:] == -9).all()


def test_seq_metadata_errors():
    import depthwise_causal_conv1d_amd as lib
    qsl = torch.tensor([0, 4], dtype=torch.int32, device=DEV)
    buf = torch.zeros(4, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="is below num_actual_tokens"):
        lib.sconv_seq_metadata(qsl, 1, 4, buf, buf.clone(), 3)
    with pytest.raises(ValueError, match="holds 3 entries"):
        lib.sconv_seq_metadata(qsl, 1, 4, buf[:3], buf.clone(), 4)


# ------------------------------------------------------------------ fused insert + conv

def check_fused(case, what, cache_compare="full", fold=False):
    """Run both sides on one case and compare out, metadata and cache."""
    say(f"fused {what}: T={case.T} C={case.C} W={case.W} N={case.block_size} "
        f"dtype={case.x.dtype} off_s={case.off_s} folded={fold}")
    out_g, cache_g, si_g, qs_g = gpu_fused(case, fold=fold)
    sm_h = to_np(case.slot_mapping)
    if cache_compare == "full":
        out_r, cache_r, si_r, qs_r = oracle_fused(case)
        cache_gh = to_np(cache_g)
    else:  # compact both sides to the referenced blocks
        cc, bt, sm = case.compact()
        sm_h = to_np(sm)
        out_r, cache_r, si_r, qs_r = oracle_fused(case, cache=cc, block_table=bt, slot_mapping=sm)
        ids = case.used_blocks.to(cache_g.device)
        cache_gh = to_np(cache_g[ids])
        # blocks nobody references must still be untouched poison
        untouched = torch.ones(cache_g.shape[0], dtype=torch.bool, device=cache_g.device)
        untouched[ids] = False
        if untouched.any():
            assert torch.isnan(cache_g[untouched].float()).all(), "write outside referenced blocks"
    if si_g is not None:
        np.testing.assert_array_equal(to_np(si_g), si_r)
        np.testing.assert_array_equal(to_np(qs_g), qs_r)
    live = live_rows(case)
    out_gh = to_np(out_g)
    assert_close(out_gh, out_r, dtype_name(case.x.dtype), f"{what} out", mask=live)
    assert_bits_equal(out_gh[~live], out_r[~live], f"{what} PAD rows untouched")
    assert_bits_equal(cache_gh, cache_r, f"{what} cache")
    assert_finite(written_cache_values(cache_gh, sm_h, case.block_size, case.off_s, case.ws),
                  f"{what} inserted cache slots")
    return out_g, cache_g


SWEEP = [
    # name, dtype, W, H, ws, D, off_s, N, new, ctx, pad, tail, act, res
    ("bf16-vec", torch.bfloat16, 4, 4, 16, 48, 16, 16, [5, 40, 1, 17, 3], [0, 70, 2, 31, 15], 6, 3, "silu", True),
    ("bf16-scalar", torch.bfloat16, 4, 3, 6, 16, 3, 16, [9, 1, 22], [4, 50, 0], 2, 0, "silu", True),
    ("f32-vec", torch.float32, 4, 2, 8, 32, 8, 16, [12, 2, 30], [1, 9, 60], 3, 2, "silu", True),
    ("f32-scalar", torch.float32, 3, 5, 3, 7, 2, 8, [6, 13], [3, 0], 1, 1, None, True),
    ("n24-nonpow2", torch.bfloat16, 4, 2, 8, 16, 0, 24, [30, 7, 1], [50, 0, 23], 2, 0, "silu", False),
    ("n1", torch.bfloat16, 4, 2, 8, 8, 0, 1, [6, 4], [5, 2], 0, 0, None, False),
    ("n32-w2", torch.bfloat16, 2, 8, 16, 64, 32, 32, [20, 1, 3], [100, 31, 0], 2, 4, "silu", True),
    ("w1", torch.float32, 1, 2, 8, 16, 8, 16, [7, 3], [9, 0], 1, 0, "silu", True),
    ("w3-f32", torch.float32, 3, 4, 4, 12, 4, 4, [11, 2, 5], [0, 7, 3], 2, 1, "silu", True),
    # minimal launches: one row with a history, one row at position 0, and
    # every row PAD (nothing may be written)
    ("single-row", torch.bfloat16, 4, 4, 16, 48, 16, 16, [1], [37], 0, 0, "silu", True),
    ("single-row-pos0", torch.bfloat16, 4, 2, 8, 16, 0, 16, [1], [0], 0, 0, "silu", True),
    ("all-pad", torch.float32, 4, 2, 8, 16, 8, 16, [3, 5], [4, 0], 8, 2, "silu", True),
]


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
@pytest.mark.parametrize("spec", SWEEP, ids=[s[0] for s in SWEEP])
def test_fused_sweep(spec, fold):
    name, dt, W, H, ws, D, off, N, new, ctx, pad, tail, act, res = spec
    case = workloads.fused_case(zlib.crc32(name.encode()) % 1000, new, ctx, H=H, D=D, ws=ws, off_s=off,
                                block_size=N, W=W, dtype=dt, pad_count=pad, tail_pad=tail,
                                activation=act, use_residual=res)
    check_fused(case, name, fold=fold)


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
@pytest.mark.parametrize("T_total,C_heads", [(4507, 32), (2000, 32), (500, 32)])
def test_fused_tile_shapes(T_total, C_heads, fold):
    """Token counts that select each rows-per-wave tile (16, 4, 1) with a
    ragged tail, several requests per tile and requests straddling tiles."""
    rng = np.random.default_rng(T_total)
    R = 23
    cuts = np.sort(rng.choice(np.arange(1, T_total), R - 1, replace=False))
    new = np.diff(np.concatenate([[0], cuts, [T_total]])).tolist()
    ctx = [int(v) for v in rng.integers(0, 300, R)]
    case = workloads.fused_case(7, new, ctx, H=C_heads, D=256, ws=128, off_s=128,
                                block_size=16, W=4, dtype=torch.bfloat16,
                                pad_count=T_total // 10, tail_pad=5)
    check_fused(case, f"tiles T={T_total}", fold=fold)


GENERATIONS = [
    # name, dtype, W, H, ws, D, off_s, N, requests, pad
    ("bf16-w4-c4096", torch.bfloat16, 4, 32, 128, 512, 128, 16, 19, 0.1),
    ("bf16-w3-n24-partial-slab", torch.bfloat16, 3, 12, 64, 128, 0, 24, 7, 0.05),
    ("bf16-w2-ragged-c", torch.bfloat16, 2, 18, 96, 96, 0, 16, 31, 0.2),
    ("bf16-w1", torch.bfloat16, 1, 16, 64, 64, 0, 16, 5, 0.1),
    ("f32-w4", torch.float32, 4, 32, 64, 128, 64, 32, 11, 0.1),
]


@pytest.mark.parametrize("spec", GENERATIONS, ids=[g[0] for g in GENERATIONS])
def test_fused_several_wave_generations(spec):
    """Prefill-shaped launches of several wave generations with per-row
    request buffers: four-row tiles whose halo rows pass between the waves
    of a workgroup through LDS.  Requests straddle tiles and workgroups,
    some start at position 0, some continue long histories, PAD rows fall
    anywhere (inside requests too), and the last slab may be partial."""
    name, dt, W, H, ws, D, off, N, R, pad = spec
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    T_total = int(rng.integers(11000, 14000))
    cuts = np.sort(rng.choice(np.arange(1, T_total), R - 1, replace=False))
    new = np.diff(np.concatenate([[0], cuts, [T_total]])).tolist()
    ctx = [0 if r % 4 == 0 else int(rng.integers(1, 3000)) for r in range(R)]
    case = workloads.fused_case(zlib.crc32(name.encode()) % 1000, new, ctx, H=H, D=D, ws=ws,
                                off_s=off, block_size=N, W=W, dtype=dt,
                                pad_count=int(T_total * pad), tail_pad=7)
    plan = gpu_plan(case)
    assert (plan["rows_per_tile"], plan["stream_x_loads"], plan["request_mode"]) == (4, 0, 0), plan
    check_fused(case, f"{name} T={case.T}")


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
def test_config_tiny_prefill(fold):
    case = workloads.tiny_prefill()
    check_fused(case, "tiny prefill (fp32)", fold=fold)


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
def test_config_batched_decode(fold):
    case = workloads.batched_decode()
    check_fused(case, "batched decode", cache_compare="compact", fold=fold)


def test_folded_search_beyond_lds():
    """5000 requests (past the 512 held in registers): the folded launch
    searches the offsets in device memory; empty requests included."""
    g = torch.Generator().manual_seed(23)
    R = 5000
    new = [int(v) for v in torch.randint(0, 3, (R,), generator=g)]
    new[-1] = max(new[-1], 1)
    ctx = [int(v) for v in torch.randint(0, 40, (R,), generator=g)]
    case = workloads.fused_case(23, new, ctx, H=2, D=16, ws=8, off_s=8, block_size=16, W=4,
                                dtype=torch.bfloat16, pad_count=7, tail_pad=3)
    check_fused(case, "5000 requests, in-memory search", fold=True)


@pytest.mark.parametrize("run_len,runs,live,lens", [(100, 2, 300, (5, 11)),
                                                    (100, 8, 1500, (1, 6)),
                                                    (600, 7, 1500, (1, 6))],
                         ids=["registers-500", "search-2300", "search-5700"])
def test_folded_empty_request_runs(run_len, runs, live, lens):
    """Runs of >= 64 empty requests between two rows of one 4-row tile.  With
    up to 512 requests the folded launch counts offsets held in registers;
    above that a wave searches device memory once and reads 64 offsets from
    its first row's request on, so a row past such a run lies beyond that
    window and must be found on its own.  Over 4096 channels (8 slabs) and
    more than 2048 rows the launch uses 4-row tiles; each run is inserted
    before a request whose first row is not a tile's first."""
    rng = np.random.default_rng(run_len + runs)
    new = [int(v) for v in rng.integers(lens[0], lens[1], live)]
    T = sum(new)
    assert T > 2048
    starts = np.cumsum([0] + new[:-1])
    cand = [r for r in range(1, live) if starts[r] % 4 != 0]
    where = sorted(rng.choice(cand, runs, replace=False).tolist(), reverse=True)
    for r in where:
        new[r:r] = [0] * run_len
    ctx = [int(v) for v in rng.integers(0, 40, len(new))]
    case = workloads.fused_case(31 + run_len, new, ctx, H=32, D=128, ws=128, off_s=0,
                                block_size=16, W=4, dtype=torch.bfloat16)
    check_fused(case, f"{len(new)} requests, runs of {run_len} empty", fold=True)


def _decode_shaped_lens(rng, R, tail):
    """Request lengths in {0, 1, 2} whose rows, tail included, number at most
    R: empty and two-row requests move rows off row t == request t."""
    new = [int(v) for v in rng.choice([0, 1, 1, 2], R)]
    while sum(new) + tail > R:
        i = new.index(max(new))
        new[i] -= 1
    return new


# name, seed, R, lens ("ones" or "mixed"), ctx max, N, W, dtype, H, ws, D, off_s, pad, tail
DECODE_ROW = [
    ("ones-narrow-table", 41, 200, "ones", 300, 16, 4, torch.bfloat16, 4, 32, 64, 32, 10, 0),
    ("mixed-rows", 42, 400, "mixed", 200, 16, 4, torch.bfloat16, 4, 32, 64, 0, 20, 3),
    ("ones-beyond-256-blocks", 43, 128, "ones", 2500, 4, 4, torch.bfloat16, 2, 64, 64, 0, 4, 0),
    ("mixed-beyond-256-blocks", 44, 256, "mixed", 2500, 4, 4, torch.bfloat16, 2, 64, 64, 0, 6, 2),
    ("w2-f32", 45, 96, "mixed", 100, 8, 2, torch.float32, 4, 8, 16, 8, 3, 1),
    ("w3-scalar", 46, 150, "ones", 120, 16, 3, torch.bfloat16, 3, 6, 16, 3, 5, 0),
    ("one-request", 47, 1, "ones", 70, 16, 4, torch.bfloat16, 2, 64, 64, 0, 0, 0),
]


@pytest.mark.parametrize("spec", DECODE_ROW, ids=[s[0] for s in DECODE_ROW])
def test_folded_decode_block_row(spec):
    """Folded launches with no more rows than requests (one-row tiles) read
    block-table row t along with the metadata and take a row's history
    blocks from it when the row is request t and its blocks lie within the
    first 256 entries; other rows look their blocks up in memory.  Cases:
    every row its own request, empty and two-row requests shifting rows off
    that guess, history past the first 256 blocks (block size 4), a table
    narrower than 256 entries, W 2 and 3, fp32, the one-channel kernels and
    PAD rows."""
    name, seed, R, lens, cmax, N, W, dt, H, ws, D, off, pad, tail = spec
    rng = np.random.default_rng(seed)
    new = [1] * R if lens == "ones" else _decode_shaped_lens(rng, R, tail)
    ctx = [int(v) for v in rng.integers(0, cmax + 1, R)]
    assert sum(new) + tail <= R
    case = workloads.fused_case(seed, new, ctx, H=H, D=D, ws=ws, off_s=off, block_size=N, W=W,
                                dtype=dt, pad_count=min(pad, sum(new)), tail_pad=tail)
    check_fused(case, f"decode-shaped {name}", fold=True)


@pytest.mark.parametrize("layout", ["search-one-row-tiles", "guess-k4-mostly-wrong"])
def test_folded_search_and_failed_guess(layout):
    """Two folded request-search paths the other shapes rarely reach: more
    than 512 requests with more rows than requests (not a multiple), so
    one-row tiles search device memory; and rows a multiple of the requests
    (k = 4) but uneven request lengths, so the guess t / 4 mostly fails and
    rows fall back to the search one by one."""
    rng = np.random.default_rng(91 if layout.startswith("search") else 92)
    if layout.startswith("search"):
        R = 600
        new = [int(v) for v in rng.choice([1, 1, 2], R)]
        assert sum(new) > R and sum(new) % R != 0
    else:
        R = 50
        new = [int(v) for v in rng.integers(1, 8, R)]
        while sum(new) != 4 * R:           # adjust to exactly 4 rows per request on average
            i = int(rng.integers(0, R))
            if sum(new) > 4 * R and new[i] > 1:
                new[i] -= 1
            elif sum(new) < 4 * R and new[i] < 7:
                new[i] += 1
    ctx = [int(v) for v in rng.integers(0, 200, R)]
    case = workloads.fused_case(93, new, ctx, H=4, D=64, ws=32, off_s=16, block_size=16, W=4,
                                dtype=torch.bfloat16, pad_count=5)
    check_fused(case, f"folded {layout}", fold=True)


def test_folded_table_needs_num_reqs_rows():
    """The folded forms may read any block-table row below num_reqs, so the
    binding refuses a shorter table before launching."""
    import depthwise_causal_conv1d_amd as lib
    case = workloads.fused_case(49, [1, 1, 1], [5, 9, 2], H=2, D=16, ws=8, block_size=16, W=4,
                                dtype=torch.bfloat16)
    x, w, cache = case.x.to(DEV), case.weight.to(DEV), case.cache.to(DEV)
    pos, sm = case.positions.to(DEV), case.slot_mapping.to(DEV)
    qsl = case.query_start_loc.to(DEV)
    bt = case.block_table.to(DEV)
    with pytest.raises(ValueError, match="num_reqs"):
        lib.sconv_fused_insert_conv_qsl(x, w, cache, pos, bt[:2], qsl, 3, sm, 0, 8, 16)
    with pytest.raises(ValueError, match="num_reqs"):
        lib.sconv_fused_insert_conv_streams([x], [w], cache, pos, bt[:2], sm, [0], [8], 16,
                                            query_start_loc=qsl, num_reqs=3)


def test_folded_decode_wide_table_stride():
    """A decode batch whose block table is a view into much wider rows: the
    guessed launch reads block-table row t ahead through the table's row
    stride, which it takes as a 32-bit leading kernel argument (here
    max_blocks + 70 000 entries; the entries past each row's first
    max_blocks are never read)."""
    import depthwise_causal_conv1d_amd as lib
    rng = np.random.default_rng(52)
    R = 96
    ctx = [int(v) for v in rng.integers(1, 1500, R)]
    case = workloads.fused_case(52, [1] * R, ctx, H=8, D=128, ws=32, block_size=16, W=4,
                                dtype=torch.bfloat16, pad_count=5)
    mb = case.block_table.shape[1]
    wide = torch.full((case.block_table.shape[0], mb + 70_000), -7, dtype=torch.int32)
    wide[:, :mb] = case.block_table
    bt = wide.to(DEV)[:, :mb]
    assert bt.stride(0) == mb + 70_000
    x, w, cache = case.x.to(DEV), case.weight.to(DEV), case.cache.to(DEV).clone()
    pos, sm = case.positions.to(DEV), case.slot_mapping.to(DEV)
    qsl = case.query_start_loc.to(DEV)
    out = torch.full_like(x, SENTINEL)
    say(f"folded decode R={R} table stride {bt.stride(0)}")
    lib.sconv_fused_insert_conv_qsl(x, w, cache, pos, bt, qsl, case.num_reqs, sm, case.off_s,
                                    case.ws, case.block_size, case.activation, case.use_residual,
                                    out=out)
    torch.cuda.synchronize()
    out_r, cache_r, _, _ = oracle_fused(case)
    live = live_rows(case)
    out_h = to_np(out)
    assert_close(out_h, out_r, "bf16", "wide-stride decode out", mask=live)
    assert_bits_equal(out_h[~live], out_r[~live], "wide-stride decode PAD rows untouched")
    assert_bits_equal(to_np(cache), cache_r, "wide-stride decode cache")


def test_streams_decode_block_row_shifted():
    """The same read-ahead in a four-stream launch, rows shifted off their
    guess by empty and two-row requests."""
    rng = np.random.default_rng(48)
    R = 300
    new = _decode_shaped_lens(rng, R, 2)
    ctx = [int(v) for v in rng.integers(0, 900, R)]
    cases = workloads.fused_streams_case(48, new, ctx, H=8, D=128,
                                         streams=[(0, 32), (32, 32), (64, 32), (96, 32)],
                                         block_size=4, W=4, dtype=torch.bfloat16,
                                         pad_count=8, tail_pad=2)
    check_streams(cases, "decode-shaped streams, shifted rows", True)


# Block size 1 000 003 (prime) with 2147 table entries: max_blocks * N is
# 2 147 006 441, just under the 2^31 the launch accepts.
_BIG_N = 1_000_003
_NEAR_MAX = [
    # name, new rows per request, positions of each request's first new row
    ("prefill-shaped", [5, 1, 3, 2], [2_147_000_000 - 5, 2146 * _BIG_N + 1, 1000 * _BIG_N + 2, 0]),
    ("decode-shaped", [1, 1, 1, 1], [2_147_000_000 - 1, 2146 * _BIG_N + 2, 255 * _BIG_N + 1, 5]),
]


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
@pytest.mark.parametrize("spec", _NEAR_MAX, ids=[s[0] for s in _NEAR_MAX])
def test_fused_positions_near_int31(spec, fold):
    """Positions up to ~2.147e9 and block indices up to 2146 with a block size
    that is not a power of two: the 32-bit position and slot arithmetic and
    the division by N at the top of their range, histories that straddle a
    block boundary, and (decode-shaped, folded) history blocks far past the
    entries a decode launch reads ahead."""
    name, new, ctx = spec
    case = workloads.fused_case(61, new, ctx, H=1, D=8, ws=8, off_s=0, block_size=_BIG_N, W=4,
                                dtype=torch.bfloat16)
    assert case.block_table.shape[1] * _BIG_N < 2 ** 31
    check_fused(case, f"positions near 2^31, {name}", fold=fold)


_STREAMS_ORACLE = {}


_KINDS = ("decode", "decode-shifted", "prefill", "spec", "empty-runs", "large")


def _random_fused_spec(k):
    """Case k of the seeded random sweep: the layout kind cycles through
    _KINDS; dtype, W, block size, heads, streams (16-byte-lane or odd widths,
    gaps between column ranges), history lengths, PAD and tail rows and the
    metadata form are drawn from a generator seeded with k."""
    rng = np.random.default_rng(4000 + k)
    kind = _KINDS[k % len(_KINDS)]
    dt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    lane = 8 if dt == torch.bfloat16 else 4
    W = int(rng.integers(1, 5))
    N = int(rng.choice([1, 4, 8, 16, 24, 32]))
    if kind == "large":
        H, nst, unit, cmax = 32, 1, lane, 600
        widths = [128 if dt == torch.bfloat16 else 64]
    else:
        H = int(rng.integers(1, 9))
        nst = int(rng.choice([1, 1, 2, 3, 4]))
        unit = lane if rng.random() < 0.75 else 1
        widths = [unit * int(rng.integers(1, 5)) for _ in range(nst)]
        cmax = int(rng.choice([0, 40, 3000]))
    offs, at = [], unit * int(rng.integers(0, 2))
    for w_ in widths:
        offs.append(at)
        at += w_ + unit * int(rng.integers(0, 2))
    D = at + unit * int(rng.integers(0, 2))
    if kind == "decode":
        R = int(rng.integers(1, 600))
        new = [1] * R
    elif kind == "decode-shifted":
        R = int(rng.integers(2, 600))
        new = _decode_shaped_lens(rng, R, 0)
    elif kind == "prefill":
        R = int(rng.integers(1, 12))
        new = [int(v) for v in rng.integers(1, 300, R)]
    elif kind == "spec":
        R = int(rng.integers(1, 300))
        new = [4] * R
    elif kind == "empty-runs":
        R = int(rng.integers(60, 700))
        new = [int(v) for v in rng.choice([0, 0, 0, 1, 3], R)]
        new[-1] = max(new[-1], 1)
    else:
        R = int(rng.integers(2, 6))
        new = [int(v) for v in rng.integers(1500, 3000, R)]
    ctx = [int(v) for v in rng.integers(0, cmax + 1, R)]
    T = sum(new)
    pad = int(rng.integers(0, T // 8 + 1))
    tail = int(rng.integers(0, 4))
    fold = bool(rng.random() < 0.5)
    return dict(kind=kind, dt=dt, W=W, N=N, H=H, D=D, streams=list(zip(offs, widths)), new=new,
                ctx=ctx, pad=pad, tail=tail, fold=fold)


@pytest.mark.parametrize("k", range(24))
def test_fused_random_sweep(k):
    """24 seeded random launches of the fused op, single- or multi-stream,
    against the oracle (outputs, PAD rows untouched, whole cache)."""
    c = _random_fused_spec(k)
    if len(c["streams"]) == 1:
        off, ws = c["streams"][0]
        case = workloads.fused_case(5000 + k, c["new"], c["ctx"], H=c["H"], D=c["D"], ws=ws,
                                    off_s=off, block_size=c["N"], W=c["W"], dtype=c["dt"],
                                    pad_count=c["pad"], tail_pad=c["tail"])
        check_fused(case, f"random {k} ({c['kind']})", fold=c["fold"])
    else:
        cases = workloads.fused_streams_case(5000 + k, c["new"], c["ctx"], H=c["H"], D=c["D"],
                                             streams=c["streams"], block_size=c["N"], W=c["W"],
                                             dtype=c["dt"], pad_count=c["pad"],
                                             tail_pad=c["tail"])
        check_streams(cases, f"random {k} ({c['kind']})", c["fold"])


def check_streams(cases, what, fold, cache_compare="full"):
    """One multi-stream launch against the oracle's multi-stream op: every
    stream's output (PAD rows untouched) and the shared cache, bit for bit."""
    c0 = cases[0]
    say(f"streams {what}: {len(cases)} streams T={c0.T} ws={[c.ws for c in cases]} "
        f"off_s={[c.off_s for c in cases]} dtype={c0.x.dtype} folded={fold}")
    outs_g, cache_g = gpu_fused_streams(cases, fold=fold)
    sm_h = to_np(c0.slot_mapping)
    if cache_compare == "full":
        if what not in _STREAMS_ORACLE:  # the same inputs serve both metadata forms
            _STREAMS_ORACLE[what] = oracle_fused_streams(cases)
        outs_r, cache_r = _STREAMS_ORACLE[what]
        cache_gh = to_np(cache_g)
    else:
        cc, bt, sm = c0.compact()
        sm_h = to_np(sm)
        outs_r, cache_r = oracle_fused_streams(cases, cache=cc, block_table=bt, slot_mapping=sm)
        cache_gh = to_np(cache_g[c0.used_blocks.to(cache_g.device)])
    live = live_rows(c0)
    for i, (og, orf) in enumerate(zip(outs_g, outs_r)):
        ogh = to_np(og)
        assert_close(ogh, orf, dtype_name(c0.x.dtype), f"{what} stream {i} out", mask=live)
        assert_bits_equal(ogh[~live], orf[~live], f"{what} stream {i} PAD rows untouched")
    assert_bits_equal(cache_gh, cache_r, f"{what} cache")
    for c in cases:
        assert_finite(written_cache_values(cache_gh, sm_h, c0.block_size, c.off_s, c.ws),
                      f"{what} inserted cache slots, columns {c.off_s}+{c.ws}")


STREAM_SPECS = [
    # name, dtype, W, H, D, N, streams (off_s, ws), acts, residuals, new, ctx, pad, tail
    ("bf16-vec", torch.bfloat16, 4, 4, 64, 16, [(0, 16), (16, 16), (32, 32)],
     ["silu", None, "silu"], [True, False, True], [9, 1, 30, 4], [20, 3, 0, 50], 4, 2),
    ("bf16-scalar", torch.bfloat16, 4, 3, 32, 8, [(0, 8), (8, 6), (20, 10)],
     ["silu", "silu", None], [True, True, False], [12, 2, 7], [0, 9, 30], 3, 1),
    ("f32-vec", torch.float32, 4, 2, 16, 16, [(0, 4), (4, 8), (12, 4)],
     [None, "silu", "silu"], [True, True, True], [5, 17], [2, 40], 2, 0),
    ("bf16-w3-two", torch.bfloat16, 3, 8, 64, 32, [(32, 32), (0, 16)],
     ["silu", "silu"], [False, True], [3, 60, 1], [100, 7, 0], 5, 3),
    ("bf16-w2-three", torch.bfloat16, 2, 4, 64, 16, [(0, 16), (16, 16), (48, 16)],
     ["silu", None, "silu"], [True, True, False], [7, 30, 2, 1], [5, 0, 40, 17], 3, 1),
]


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
@pytest.mark.parametrize("spec", STREAM_SPECS, ids=[s[0] for s in STREAM_SPECS])
def test_streams_sweep(spec, fold):
    name, dt, W, H, D, N, streams, acts, ress, new, ctx, pad, tail = spec
    cases = workloads.fused_streams_case(zlib.crc32(name.encode()) % 1000, new, ctx, H=H, D=D,
                                         streams=streams, block_size=N, W=W, dtype=dt,
                                         pad_count=pad, tail_pad=tail, activations=acts,
                                         residuals=ress)
    check_streams(cases, name, fold)


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
def test_streams_mixed_prefill_one_launch(fold):
    """The four streams of the mixed prefill (ws 128 at off_s 0/128/256/384 of
    D=512, 20 450 rows, 10% PAD) in one launch."""
    check_streams(workloads.mixed_prefill_streams(), "mixed prefill", fold)


def test_streams_decode_layer():
    """A decode batch of 256 requests with all four streams of the layer
    (ws=32 each, D=128) in one folded launch."""
    g = torch.Generator().manual_seed(5)
    ctx = [int(v) for v in torch.randint(1, 4097, (256,), generator=g)]
    cases = workloads.fused_streams_case(5, [1] * 256, ctx, H=32, D=128,
                                         streams=[(0, 32), (32, 32), (64, 32), (96, 32)],
                                         block_size=16, W=4, dtype=torch.bfloat16)
    check_streams(cases, "decode layer", True, cache_compare="compact")


def test_streams_spec_decode_four_row_tiles():
    """A layer's speculative step in one folded launch: 512 requests x 4
    drafts over four streams (ws=128 each, D=512), enough waves for
    four-row tiles, where each tile's rows are checked against the guess
    t / 4."""
    g = torch.Generator().manual_seed(94)
    ctx = [int(v) for v in torch.randint(1, 2000, (512,), generator=g)]
    cases = workloads.fused_streams_case(94, [4] * 512, ctx, H=8, D=512,
                                         streams=[(0, 128), (128, 128), (256, 128), (384, 128)],
                                         block_size=16, W=4, dtype=torch.bfloat16, pad_count=20)
    check_streams(cases, "spec decode, four streams", True, cache_compare="compact")


def test_streams_one_stream_equals_single_entry():
    """A one-stream call gives the same bits as sconv_fused_insert_conv."""
    case = workloads.batched_decode(seed=9)
    a_out, a_cache, _, _ = gpu_fused(case, fold=True)
    b_outs, b_cache = gpu_fused_streams([case], fold=True)
    assert_bits_equal(to_np(b_outs[0]), to_np(a_out), "out")
    assert torch.equal(b_cache.view(torch.int16), a_cache.view(torch.int16))


def test_config_batched_decode_large_pool():
    """Same decode batch with its blocks scattered over a 16k-block pool."""
    case = workloads.batched_decode(pool_blocks=16384, device=DEV)
    check_fused(case, "batched decode, large pool", cache_compare="compact")


def test_config_mixed_prefill_four_streams():
    """Four streams convolved in turn over one shared cache, 10% PAD rows."""
    streams = workloads.mixed_prefill_streams()
    import depthwise_causal_conv1d_amd as lib
    import oracle
    base = streams[0]
    say(f"mixed prefill T={base.T} C={base.C} blocks={base.cache.shape[0]}")
    cache_g = base.cache.to(DEV).clone()
    qsl = base.query_start_loc.to(DEV)
    si = torch.empty(base.T, dtype=torch.int32, device=DEV)
    qs = torch.empty_like(si)
    lib.sconv_seq_metadata(qsl, base.num_reqs, base.num_actual, si, qs, base.T)
    pos, bt, sm = base.positions.to(DEV), base.block_table.to(DEV), base.slot_mapping.to(DEV)
    si_r, qs_r = oracle.seq_metadata(to_np(base.query_start_loc), base.num_reqs,
                                     base.num_actual, base.T)
    cache_r = to_np(base.cache)
    live = live_rows(base)
    for s, case in enumerate(streams):
        out_g = torch.full_like(case.x, SENTINEL, device=DEV)
        lib.sconv_fused_insert_conv(case.x.to(DEV), case.weight.to(DEV), cache_g, pos, bt, si,
                                    sm, qs, case.off_s, case.ws, case.block_size, "silu", True,
                                    out=out_g)
        out_r, cache_r = oracle.fused_insert_conv(
            to_np(case.x), to_np(case.weight), cache_r, to_np(base.positions),
            to_np(base.block_table), si_r, to_np(base.slot_mapping), qs_r, case.off_s, case.ws,
            case.block_size, "silu", True, out_init=np.full(case.x.shape, 0xC442, np.uint16))
        out_h = to_np(out_g)
        assert_close(out_h, out_r, "bf16", f"stream {s}", mask=live)
        assert (out_h[~live] == 0xC442).all()   # bf16 bits of -777
        say(f"  stream {s} ok")
    cache_h = to_np(cache_g)
    assert_bits_equal(cache_h, cache_r, "shared cache after four streams")
    for case in streams:
        assert_finite(written_cache_values(cache_h, to_np(base.slot_mapping), base.block_size,
                                           case.off_s, case.ws), f"stream at {case.off_s} inserts")


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
def test_config_spec_decode(fold):
    case = workloads.spec_decode()
    check_fused(case, "spec decode", cache_compare="compact", fold=fold)


# ------------------------------------------------------------------ hipGraph replay

def test_graph_replay_folded_decode_layouts():
    """One captured folded decode launch (48 rows, 48 requests), replayed on
    three request layouts written into its buffers: every row its own
    request (the request guess holds), empty and two-row requests with
    padded tail rows (rows off the guess), and histories past the first 256
    block-table entries.  The choice between these paths is made on the
    device at each replay; every replay equals the oracle, outputs and the
    whole cache."""
    import depthwise_causal_conv1d_amd as lib
    R, N, H, D, ws, WBT, POOL = 48, 4, 4, 64, 32, 400, 128
    rng = np.random.default_rng(71)
    mixed = _decode_shaped_lens(rng, R, 4)
    layouts = [("one row per request", [1] * R, [int(v) for v in rng.integers(0, 300, R)]),
               ("empty and two-row requests", mixed, [int(v) for v in rng.integers(0, 300, R)]),
               ("histories past 256 blocks", [1] * R,
                [int(v) for v in rng.integers(1000, 1590, R)])]
    cases = []
    for k, (name, new, ctx) in enumerate(layouts):
        c = workloads.fused_case(72 + k, new, ctx, H=H, D=D, ws=ws, block_size=N, W=4,
                                 dtype=torch.bfloat16, pool_blocks=POOL, pad_count=2,
                                 tail_pad=R - sum(new))
        assert c.T == R and c.block_table.shape[1] <= WBT
        bt = torch.full((R, WBT), c.poison_block, dtype=torch.int32)
        bt[:, :c.block_table.shape[1]] = c.block_table
        cases.append((name, c, bt))
    c0 = cases[0][1]
    x_b = torch.zeros(R, c0.C, dtype=torch.bfloat16, device=DEV)
    w_b = torch.zeros_like(c0.weight, device=DEV)
    cache_b = torch.zeros_like(c0.cache, device=DEV)
    pos_b = torch.zeros(R, dtype=torch.int64, device=DEV)
    sm_b = torch.zeros(R, dtype=torch.int64, device=DEV)
    qsl_b = torch.zeros(R + 1, dtype=torch.int32, device=DEV)
    bt_b = torch.zeros(R, WBT, dtype=torch.int32, device=DEV)
    out_b = torch.zeros_like(x_b)

    def load(c, bt):
        for dst, src in ((x_b, c.x), (w_b, c.weight), (cache_b, c.cache), (pos_b, c.positions),
                         (sm_b, c.slot_mapping), (qsl_b, c.query_start_loc), (bt_b, bt)):
            dst.copy_(src.to(DEV))
        out_b.fill_(SENTINEL)

    def step():
        lib.sconv_fused_insert_conv_qsl(x_b, w_b, cache_b, pos_b, bt_b, qsl_b, R, sm_b, 0, ws, N,
                                        "silu", True, out=out_b)

    load(c0, cases[0][2])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for name, c, bt in cases + cases[:1]:
        load(c, bt)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_r, cache_r, _, _ = oracle_fused(c)
        live = live_rows(c)
        got = to_np(out_b)
        assert_close(got, out_r, "bf16", f"{name} out", mask=live)
        assert_bits_equal(got[~live], out_r[~live], f"{name} PAD rows untouched")
        assert_bits_equal(to_np(cache_b), cache_r, f"{name} cache")
        assert_finite(written_cache_values(to_np(cache_b), to_np(c.slot_mapping), N, 0, ws),
                      f"{name} inserted cache slots")
        say(f"  replay '{name}' ok")


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
def test_graph_replay_decode_steps(fold):
    """Capture metadata + fused conv once for a decode batch; replay it for
    successive steps with new inputs written into the captured buffers.
    Each replay must equal the oracle; each step reads the previous steps'
    cache writes."""
    import depthwise_causal_conv1d_amd as lib
    R, S = 64, 6
    g = torch.Generator().manual_seed(17)
    ctx = [int(v) for v in torch.randint(1, 700, (R,), generator=g)]
    case = workloads.fused_case(17, [S] * R, ctx, H=8, D=64, ws=32, off_s=32, block_size=16,
                                W=4, dtype=torch.bfloat16)
    ref_out, ref_cache, _, _ = oracle_fused(case)     # one S-token call == S steps
    qsl_h = case.query_start_loc
    rows = lambda s: (qsl_h[:-1] + s).long()
    x_b = torch.zeros(R, case.C, dtype=torch.bfloat16, device=DEV)
    pos_b = torch.zeros(R, dtype=torch.int64, device=DEV)
    sm_b = torch.zeros(R, dtype=torch.int64, device=DEV)
    qsl_b = torch.arange(R + 1, dtype=torch.int32, device=DEV)
    si_b = torch.zeros(R, dtype=torch.int32, device=DEV)
    qs_b = torch.zeros(R, dtype=torch.int32, device=DEV)
    out_b = torch.zeros_like(x_b)
    w = case.weight.to(DEV)
    cache = case.cache.to(DEV).clone()
    bt = case.block_table.to(DEV)

    def step():
        if fold:
            lib.sconv_fused_insert_conv_qsl(x_b, w, cache, pos_b, bt, qsl_b, R, sm_b, case.off_s,
                                            case.ws, case.block_size, "silu", True, out=out_b)
            return
        lib.sconv_seq_metadata(qsl_b, R, R, si_b, qs_b, R)
        lib.sconv_fused_insert_conv(x_b, w, cache, pos_b, bt, si_b, sm_b, qs_b, case.off_s,
                                    case.ws, case.block_size, "silu", True, out=out_b)

    def load(s):
        x_b.copy_(case.x[rows(s)].to(DEV))
        pos_b.copy_(case.positions[rows(s)].to(DEV))
        sm_b.copy_(case.slot_mapping[rows(s)].to(DEV))

    # warm up on a side stream, then restore the cache
    cache0 = cache.clone()
    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cache.copy_(cache0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    cache.copy_(cache0)
    for s in range(S):
        load(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_close(to_np(out_b), ref_out[rows(s).numpy()], "bf16", f"replay {s}")
        say(f"  replay {s} ok")
    assert_bits_equal(to_np(cache), ref_cache, "cache after replays")
    assert_finite(written_cache_values(to_np(cache), to_np(case.slot_mapping), case.block_size,
                                       case.off_s, case.ws), "inserted cache slots")


def test_graph_replay_batched_decode_full_size():
    """The benchmarked decode step at full size, captured once and replayed
    on three batches written into its buffers in place: 256 requests x 1
    token, histories uniform in [1, 4096], H=32, D=128, ws=32 (C=1024), N=16,
    bf16, SiLU and residual, request search folded into the launch.  The
    three batches own disjoint blocks of one shared pool.  After each replay
    the outputs equal the oracle within tolerance and every block the batch
    references equals it bit for bit; after the last, every block no batch
    references is still NaN poison."""
    import depthwise_causal_conv1d_amd as lib
    B, NB = 256, 3
    full = workloads.batched_decode(device=DEV, num_reqs=B * NB,
                                    pool_blocks=int(B * NB * 2 * 1.25) + 1)
    say(f"full-size decode graph: {NB} batches of {B}, pool {full.cache.shape[0]} blocks")
    cache = full.cache                       # device, shared by the batches
    x_b = torch.zeros(B, full.C, dtype=torch.bfloat16, device=DEV)
    pos_b = torch.zeros(B, dtype=torch.int64, device=DEV)
    sm_b = torch.full((B,), -1, dtype=torch.int64, device=DEV)
    bt_b = torch.zeros(B, full.block_table.shape[1], dtype=torch.int32, device=DEV)
    qsl_b = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    out_b = torch.zeros_like(x_b)
    w = full.weight.to(DEV)

    def step():
        lib.sconv_fused_insert_conv_qsl(x_b, w, cache, pos_b, bt_b, qsl_b, B, sm_b, full.off_s,
                                        full.ws, full.block_size, "silu", True, out=out_b)

    # warm-up launch on all-PAD rows (nothing is written), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    assert torch.isnan(cache.float()).sum() > 0
    for i in range(NB):
        rows = slice(i * B, (i + 1) * B)
        sub = full.select(rows, rows)
        cc, bt_c, sm_c = sub.compact()
        out_r, cache_r, _, _ = oracle_fused(sub, cache=cc, block_table=bt_c, slot_mapping=sm_c)
        x_b.copy_(sub.x.to(DEV))
        pos_b.copy_(sub.positions.to(DEV))
        sm_b.copy_(sub.slot_mapping.to(DEV))
        bt_b.copy_(sub.block_table.to(DEV))
        out_b.fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_close(to_np(out_b), out_r, "bf16", f"batch {i} out")
        got = to_np(cache[sub.used_blocks.to(DEV)])
        assert_bits_equal(got, cache_r, f"batch {i} referenced blocks")
        assert_finite(written_cache_values(got, to_np(sm_c), sub.block_size, 0, sub.ws),
                      f"batch {i} inserted slots")
        say(f"  replay of batch {i} ok")
    untouched = torch.ones(cache.shape[0], dtype=torch.bool, device=DEV)
    untouched[full.used_blocks.to(DEV)] = False
    assert untouched.any()
    assert torch.isnan(cache[untouched].float()).all(), "write outside the referenced blocks"


# ------------------------------------------------------------------ SSM-style ops

def gpu_varlen(case, inplace=False):
    import depthwise_causal_conv1d_amd as lib
    x = case.x.to(DEV)
    st = case.conv_states.to(DEV).clone()
    out = x.clone() if inplace else torch.full_like(x, SENTINEL)
    xin = out if inplace else x
    lib.causal_conv1d_varlen_fwd(
        xin, case.weight.to(DEV), None if case.bias is None else case.bias.to(DEV), st,
        case.query_start_loc.to(DEV),
        None if case.cache_indices is None else case.cache_indices.to(DEV),
        None if case.has_initial_state is None else case.has_initial_state.to(DEV),
        case.activation == "silu", case.pad_slot_id, out=out)
    return out, st


def oracle_varlen(case):
    import oracle
    return oracle.causal_conv1d_varlen_fwd(
        to_np(case.x), to_np(case.weight), None if case.bias is None else to_np(case.bias),
        to_np(case.conv_states), to_np(case.query_start_loc),
        None if case.cache_indices is None else to_np(case.cache_indices),
        None if case.has_initial_state is None else to_np(case.has_initial_state),
        case.activation, case.pad_slot_id, out_init=_sentinel_like(case.x))


def _sentinel_like(t):
    return to_np(torch.full_like(t, SENTINEL))


VARLEN = [
    # name, dtype, lens, dim, W, init, pad, bias, act, x_padding
    ("bf16-aligned", torch.bfloat16, [64, 128, 512, 8], 24, 4, 2, 0, 0.1, "silu", 0),
    ("bf16-ragged", torch.bfloat16, [13, 1, 0, 700, 2, 91], 10, 4, 3, 1, 0.1, "silu", 0),
    ("bf16-xpad", torch.bfloat16, [37, 200, 5], 16, 4, 1, 0, None, None, 11),
    ("f32-ragged", torch.float32, [5, 300, 17, 1], 12, 4, 2, 1, 0.2, "silu", 0),
    ("f32-w3", torch.float32, [9, 66], 8, 3, 1, 0, 0.2, "silu", 0),
    ("bf16-w2", torch.bfloat16, [1, 9, 130], 8, 2, 2, 0, 0.1, None, 0),
    ("bf16-w1", torch.bfloat16, [4, 20], 8, 1, 1, 0, 0.1, "silu", 0),
]


@pytest.mark.parametrize("spec", VARLEN, ids=[v[0] for v in VARLEN])
def test_varlen_sweep(spec):
    name, dt, lens, dim, W, init, pad, bias, act, xpad = spec
    case = workloads.varlen_case(zlib.crc32(name.encode()) % 1000, lens, dim=dim, num_slots=len(lens) + 5, W=W,
                                 dtype=dt, init_count=init, pad_seqs=pad, bias_std=bias,
                                 activation=act, x_padding=xpad)
    say(f"varlen {name}")
    out_r, st_r = oracle_varlen(case)
    for inplace in (False, True):
        out_g, st_g = gpu_varlen(case, inplace=inplace)
        ci = to_np(case.cache_indices)
        qsl = to_np(case.query_start_loc)
        mask = np.zeros(case.x.shape, bool)
        for b in range(len(lens)):
            if ci[b] != case.pad_slot_id:
                mask[:, qsl[b]:qsl[b + 1]] = True
        og = to_np(out_g)
        assert_close(og, out_r, dtype_name(dt), f"{name} out inplace={inplace}", mask=mask)
        if not inplace:
            assert_bits_equal(og[~mask], out_r[~mask], "PAD sequences untouched")
        assert_bits_equal(to_np(st_g), st_r, f"{name} states inplace={inplace}")
        assert_finite(to_np(st_g)[ci[ci != case.pad_slot_id]], f"{name} written states")


def test_varlen_transposed_view_and_null_options():
    """x given as a transposed view (token stride != 1): the scalar path;
    no cache_indices / has_initial_state (slot b, zero history)."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(3)
    base = torch.randn(90, 12, generator=g).to(torch.bfloat16)      # [T, dim]
    x = base.T                                                       # [dim, T] view
    w = (torch.randn(12, 4, generator=g) * 0.5).to(torch.bfloat16)
    st = torch.full((3, 12, 3), float("nan"), dtype=torch.bfloat16)
    qsl = torch.tensor([0, 40, 41, 90], dtype=torch.int32)
    out_r, st_r = oracle.causal_conv1d_varlen_fwd(to_np(x), to_np(w), None, to_np(st),
                                                  to_np(qsl), None, None, "silu", -1)
    xd = base.to(DEV).T
    std = st.to(DEV)
    out_g = torch.empty(12, 90, dtype=torch.bfloat16, device=DEV)
    lib.causal_conv1d_varlen_fwd(xd, w.to(DEV), None, std, qsl.to(DEV), None, None, True, -1,
                                 out=out_g)
    assert_close(to_np(out_g), out_r, "bf16", "transposed view")
    assert_bits_equal(to_np(std), st_r, "states")


def test_config_ssm_varlen_and_updates():
    """8 x 4096 tokens, dim 8192, pool of 1024 slots, then 64 decode steps."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    case = workloads.ssm_varlen()
    say("ssm varlen: oracle")
    out_r, st_r = oracle_varlen(case)
    say("ssm varlen: gpu")
    out_g, st_g = gpu_varlen(case)
    assert_close(to_np(out_g), out_r, "bf16", "ssm varlen out")
    assert_bits_equal(to_np(st_g), st_r, "ssm varlen states")
    assert_finite(to_np(st_g)[to_np(case.cache_indices)], "ssm varlen written states")
    out_i, st_i = gpu_varlen(case, inplace=True)
    assert_bits_equal(to_np(out_i), to_np(out_g), "in-place == out-of-place")
    assert_bits_equal(to_np(st_i), to_np(st_g), "in-place states")
    del out_i, st_i
    say("ssm updates")
    xs = workloads.update_inputs(3, 64, 8, 8192)
    ci = case.cache_indices
    w, b = case.weight, case.bias
    st_cpu = st_r
    wd, bd, cid = w.to(DEV), b.to(DEV), ci.to(DEV)
    y_ref = []
    for s, xs_s in enumerate(xs):
        y_r, st_cpu = oracle.causal_conv1d_update(to_np(xs_s), st_cpu, to_np(w), to_np(b), "silu",
                                                  to_np(ci), -1)
        y_ref.append(y_r)
        y_g = lib.causal_conv1d_update(xs_s.to(DEV), st_g, wd, bd, True, None, cid, -1,
                                       out=torch.empty(8, 8192, dtype=torch.bfloat16, device=DEV))
        assert_close(to_np(y_g), y_r, "bf16", f"update step {s}")
    assert_bits_equal(to_np(st_g), st_cpu, "states after 64 updates")
    assert_finite(to_np(st_g)[to_np(ci)], "live states after 64 updates")

    # The same 64 steps captured as one hipGraph, replayed on the pool as the
    # prefill left it: every step's output and the final pool as above.
    say("ssm updates: 64 steps in one graph")
    st_p = np.ascontiguousarray(st_r)
    pool = torch.from_numpy(st_p.view(np.int16)).view(torch.bfloat16).to(DEV)
    x_all = torch.stack(xs).to(DEV)
    y_all = torch.full_like(x_all, SENTINEL)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a scratch copy of the pool
        scratch = pool.clone()
        lib.causal_conv1d_update(x_all[0], scratch, wd, bd, True, None, cid, -1,
                                 out=torch.empty_like(x_all[0]))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del scratch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(len(xs)):
            lib.causal_conv1d_update(x_all[s], pool, wd, bd, True, None, cid, -1, out=y_all[s])
    torch.cuda.synchronize()
    assert_bits_equal(to_np(pool), st_p, "pool untouched by the capture")
    graph.replay()
    torch.cuda.synchronize()
    for s in range(len(xs)):
        assert_close(to_np(y_all[s]), y_ref[s], "bf16", f"graph step {s}")
    assert_bits_equal(to_np(pool), st_cpu, "states after the 64-step graph")


@pytest.mark.parametrize("dt,W,dim,idx,inplace", [
    (torch.bfloat16, 4, 64, True, False), (torch.bfloat16, 4, 60, True, True),
    (torch.float32, 4, 32, False, False), (torch.float32, 2, 10, True, True),
    (torch.bfloat16, 3, 40, True, False), (torch.bfloat16, 1, 16, True, False),
    # odd dims: the one-channel kernel
    (torch.bfloat16, 4, 37, True, False), (torch.float32, 3, 13, False, True)])
def test_update_sweep(dt, W, dim, idx, inplace):
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(dim * 10 + W)
    batch, slots = 7, 11
    x = torch.randn(batch, dim, generator=g).to(dt)
    w = (torch.randn(dim, W, generator=g) * 0.5).to(dt)
    b = (torch.randn(dim, generator=g) * 0.1).to(dt)
    st = torch.randn(slots, dim, W - 1, generator=g).to(dt)
    ci = torch.randperm(slots, generator=g)[:batch].to(torch.int32)
    ci[3] = -1
    if not idx:
        ci = None
    out_r, st_r = oracle.causal_conv1d_update(to_np(x), to_np(st), to_np(w), to_np(b), "silu",
                                              None if ci is None else to_np(ci), -1,
                                              out_init=_sentinel_like(x))
    xd = x.to(DEV)
    std = st.to(DEV)
    out = xd if inplace else torch.full_like(xd, SENTINEL)
    lib.causal_conv1d_update(xd, std, w.to(DEV), b.to(DEV), True, None,
                             None if ci is None else ci.to(DEV), -1, out=out)
    live = np.ones(batch, bool)
    if ci is not None:
        live[3] = False
    assert_close(to_np(out), out_r, dtype_name(dt), "update out", mask=live)
    if not inplace and ci is not None:
        assert_bits_equal(to_np(out)[3], out_r[3], "PAD row untouched")
    assert_bits_equal(to_np(std), st_r, "states")
    assert_finite(to_np(std), "states")


# ------------------------------------------------------------------ gather

@pytest.mark.parametrize("real_count", [0, 1, 256, 512, 600, -4])
def test_config_spec_gather(real_count):
    import depthwise_causal_conv1d_amd as lib
    import oracle
    case = workloads.spec_decode()
    gc = workloads.spec_gather(case, real_count=real_count)
    say(f"gather real_count={real_count}")
    out_r = oracle.gather_conv_window(to_np(gc.src), to_np(gc.abs_positions), gc.real_count,
                                      to_np(gc.out_init), gc.d_conv)
    out_g = gc.out_init.to(DEV).clone()
    rc = torch.tensor([gc.real_count], dtype=torch.int32, device=DEV)
    lib.gather_intermediate_conv_window(gc.src.to(DEV), gc.abs_positions.to(DEV), rc, out_g,
                                        gc.d_conv)
    assert_bits_equal(to_np(out_g), out_r, "gathered windows")
    assert_finite(to_np(out_g)[:max(0, min(real_count, 512))], "live gathered windows")


@pytest.mark.parametrize("dt,conv_dim,d_conv,seq_len", [
    (torch.bfloat16, 24, 3, 50), (torch.float32, 12, 4, 9), (torch.bfloat16, 7, 2, 30),
    (torch.float32, 5, 1, 3)])
def test_gather_sweep(dt, conv_dim, d_conv, seq_len):
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(conv_dim)
    src = torch.randn(1, seq_len, conv_dim, generator=g).to(dt)
    mc = 19
    pos = torch.randint(-3, seq_len + 5, (mc,), generator=g).to(torch.int32)
    out0 = torch.full((mc, conv_dim, d_conv), SENTINEL).to(dt)
    for n in (0, 7, mc):
        out_r = oracle.gather_conv_window(to_np(src), to_np(pos), n, to_np(out0), d_conv)
        out_g = out0.to(DEV).clone()
        lib.gather_intermediate_conv_window(src.to(DEV), pos.to(DEV),
                                            torch.tensor([n], dtype=torch.int32, device=DEV),
                                            out_g, d_conv)
        assert_bits_equal(to_np(out_g), out_r, f"gather n={n}")


def test_gather_graph_replay_with_device_count():
    """Grid fixed at capture (max_count); the live count changes between
    replays through the fixed device buffer only."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    case = workloads.spec_decode()
    gc = workloads.spec_gather(case, real_count=0)
    src = gc.src.to(DEV)
    pos = gc.abs_positions.to(DEV)
    rc = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = gc.out_init.to(DEV).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.gather_intermediate_conv_window(src, pos, rc, out, 3)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.gather_intermediate_conv_window(src, pos, rc, out, 3)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(99)
    for n in [0, 512, 3] + [int(v) for v in torch.randint(0, 513, (4,), generator=g)]:
        out.copy_(gc.out_init.to(DEV))
        rc.fill_(n)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_r = oracle.gather_conv_window(to_np(gc.src), to_np(gc.abs_positions), n,
                                          to_np(gc.out_init), 3)
        assert_bits_equal(to_np(out), out_r, f"replay n={n}")


# ------------------------------------------------------------------ conv + gather, one launch

def check_conv_gather(cases, gc, what, fold=True, expect_mode=1, own_src=False):
    """sconv_fused_insert_conv_gather against the oracle's two ops: every
    stream's output, the cache (referenced blocks bit for bit, the others
    still NaN), and the gathered windows bit for bit (dead slots keep their
    sentinel).  The gather reads the first stream's x, or with own_src its
    own gc.src.  expect_mode None accepts either launch form; the form
    taken is returned."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    c0 = cases[0]
    say(f"conv+gather {what}: {len(cases)} streams T={c0.T} C={c0.C} "
        f"real_count={gc.real_count} d_conv={gc.d_conv} folded={fold}")
    xs = [c.x.to(DEV) for c in cases]
    ws_ = [c.weight.to(DEV) for c in cases]
    cache = c0.cache.to(DEV).clone()
    pos, bt, sm = c0.positions.to(DEV), c0.block_table.to(DEV), c0.slot_mapping.to(DEV)
    qsl = c0.query_start_loc.to(DEV)
    outs = [torch.full_like(x, SENTINEL) for x in xs]
    src = gc.src.to(DEV) if own_src else xs[0].view(1, c0.T, c0.C)
    gpos = gc.abs_positions.to(DEV)
    rc = torch.tensor([gc.real_count], dtype=torch.int32, device=DEV)
    gout = gc.out_init.to(DEV).clone()
    kw = dict(activation=[c.activation for c in cases],
              use_residual=[c.use_residual for c in cases], outs=outs)
    if fold:
        kw.update(query_start_loc=qsl, num_reqs=c0.num_reqs)
    else:
        si = torch.empty(c0.T, dtype=torch.int32, device=DEV)
        qs = torch.empty_like(si)
        lib.sconv_seq_metadata(qsl, c0.num_reqs, c0.num_actual, si, qs, c0.T)
        kw.update(seq_idx=si, query_start=qs)
    args = (xs, ws_, cache, pos, bt, sm, [c.off_s for c in cases], [c.ws for c in cases],
            c0.block_size)
    plan = lib.sconv_fused_plan(*args, gather=(src, gpos, rc, gout, gc.d_conv), **kw)
    if expect_mode is not None:
        assert plan["gather_mode"] == expect_mode, plan
    n = max(0, min(gc.real_count, gc.out_init.shape[0]))
    assert plan["gather_mode"] in ((1, 2) if n or gc.out_init.shape[0] else (0,)), plan
    lib.sconv_fused_insert_conv_gather(*args, src, gpos, rc, gout, gc.d_conv, **kw)
    torch.cuda.synchronize()
    cc, btc, smc = c0.compact()
    outs_r, cache_r = oracle_fused_streams(cases, cache=cc, block_table=btc, slot_mapping=smc)
    live = live_rows(c0)
    for i, (og, orf) in enumerate(zip(outs, outs_r)):
        ogh = to_np(og)
        assert_close(ogh, orf, dtype_name(c0.x.dtype), f"{what} stream {i} out", mask=live)
        assert_bits_equal(ogh[~live], orf[~live], f"{what} stream {i} PAD rows untouched")
    ids = c0.used_blocks.to(DEV)
    got = to_np(cache[ids])
    assert_bits_equal(got, cache_r, f"{what} referenced blocks")
    untouched = torch.ones(cache.shape[0], dtype=torch.bool, device=DEV)
    untouched[ids] = False
    if untouched.any():
        assert torch.isnan(cache[untouched].float()).all(), "write outside referenced blocks"
    g_r = oracle.gather_conv_window(to_np(gc.src), to_np(gc.abs_positions), gc.real_count,
                                    to_np(gc.out_init), gc.d_conv)
    g_h = to_np(gout)
    assert_bits_equal(g_h, g_r, f"{what} gathered windows")
    assert_finite(g_h[:n], f"{what} live gathered windows")
    return plan["gather_mode"]


@pytest.mark.parametrize("real_count", [0, 1, 256, 512, 600, -4])
def test_spec_step_in_one_launch(real_count):
    """The benchmarked speculative step at full size (512 requests x 4
    drafts, C=4096, N=32, bf16) with the window gather of its x (max_count
    512, d_conv 3) in the conv's launch."""
    case = workloads.spec_decode()
    gc = workloads.spec_gather(case, real_count=real_count)
    check_conv_gather([case], gc, f"spec step, {real_count} live")


@pytest.mark.parametrize("fold", [False, True], ids=["meta", "qsl"])
def test_conv_gather_four_streams_f32_and_small_windows(fold):
    """Four streams in one launch with the gather (one generation of
    four-row tiles), and an fp32 launch with d_conv 1, 2 and 4."""
    g = torch.Generator().manual_seed(95)
    ctx = [int(v) for v in torch.randint(1, 2000, (512,), generator=g)]
    cases = workloads.fused_streams_case(95, [4] * 512, ctx, H=8, D=512,
                                         streams=[(0, 128), (128, 128), (256, 128), (384, 128)],
                                         block_size=16, W=4, dtype=torch.bfloat16, pad_count=20)
    gc = workloads.gather_case(96, cases[0].x.view(1, cases[0].T, cases[0].C), max_count=300,
                               d_conv=3)
    check_conv_gather(cases, gc, "four streams", fold=fold)
    for dc, W in ((1, 4), (2, 3), (4, 2)):
        # 1024 requests x 4 rows of 1024 fp32 channels: 4096 waves of four-row tiles
        ctx = [int(v) for v in torch.randint(1, 500, (1024,), generator=g)]
        c = workloads.fused_case(97 + dc, [4] * 1024, ctx, H=16, D=96, ws=64, off_s=16,
                                 block_size=16, W=W, dtype=torch.float32, pad_count=9)
        gc = workloads.gather_case(98 + dc, c.x.view(1, c.T, c.C), max_count=200, d_conv=dc)
        check_conv_gather([c], gc, f"f32 W={W} d_conv={dc}", fold=fold)


_CG_MODES = {}


@pytest.mark.parametrize("k", range(12))
def test_conv_gather_random_sweep(k):
    """12 seeded random conv + gather launches against the oracle's two ops.
    Even cases have the one-generation shape that runs the gather in the
    conv's launch (1024-1280 requests x 4 rows, four 16-byte-lane slabs per
    row); odd ones reuse the random fused layouts, which mostly launch the
    gather after the conv.  Dtype, W, streams, metadata form, window length,
    slot count, live count (also negative or past the slots) and the
    gather's source (the conv's x or a tensor of its own) are drawn per
    case."""
    rng = np.random.default_rng(7000 + k)
    if k % 2 == 0:
        dt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
        lane = 8 if dt == torch.bfloat16 else 4
        R = int(rng.integers(1024, 1281))
        nst = int(rng.choice([1, 2]))
        ws = 64 * lane // nst if dt == torch.bfloat16 else 128 // nst
        H = 4 * 64 * lane // (ws * nst) // 1
        c = dict(kind="one-generation", dt=dt, W=int(rng.integers(1, 5)),
                 N=int(rng.choice([8, 16, 32])), H=H, D=ws * nst,
                 streams=[(i * ws, ws) for i in range(nst)], new=[4] * R,
                 ctx=[int(v) for v in rng.integers(0, 3000, R)], pad=int(rng.integers(0, 40)),
                 tail=0, fold=bool(rng.random() < 0.5))
    else:
        c = _random_fused_spec(k)
    cases = workloads.fused_streams_case(7100 + k, c["new"], c["ctx"], H=c["H"], D=c["D"],
                                         streams=c["streams"], block_size=c["N"], W=c["W"],
                                         dtype=c["dt"], pad_count=c["pad"], tail_pad=c["tail"])
    c0 = cases[0]
    own = bool(rng.random() < 0.4)
    dc = int(rng.integers(1, 5))
    if own:
        S, Cg = int(rng.integers(1, 3000)), int(rng.choice([8, 24, 40, 1024]))
        src = torch.randn(1, S, Cg, generator=torch.Generator().manual_seed(k)).to(c["dt"])
    else:
        src = c0.x.view(1, c0.T, c0.C)
    mc = int(rng.integers(1, 600))
    stride = max(1, src.shape[1] // mc)
    rc = int(rng.choice([0, 1, mc // 2, mc, mc + 7, -3]))
    gc = workloads.gather_case(7200 + k, src, max_count=mc, d_conv=dc, stride=stride,
                               real_count=rc)
    mode = check_conv_gather(cases, gc, f"random {k} ({c['kind']})", fold=c["fold"],
                             expect_mode=None, own_src=own)
    _CG_MODES[k] = mode
    if k == 10:  # the even cases so far must have run in one launch
        assert all(_CG_MODES[j] == 1 for j in _CG_MODES if j % 2 == 0), _CG_MODES


def test_conv_gather_falls_back_to_two_launches():
    """Shapes without a combined kernel (one-row decode tiles; a one-channel
    conv) launch the gather after the conv, with the same results."""
    case = workloads.batched_decode(seed=21)
    gc = workloads.gather_case(22, case.x.view(1, case.T, case.C), max_count=100, d_conv=3,
                               stride=2)
    check_conv_gather([case], gc, "decode shape", expect_mode=2)
    c = workloads.fused_case(23, [4] * 64, [5] * 64, H=3, D=16, ws=6, off_s=2, block_size=8,
                             W=4, dtype=torch.bfloat16)
    gc = workloads.gather_case(24, c.x.view(1, c.T, c.C), max_count=40, d_conv=3, stride=4)
    check_conv_gather([c], gc, "one-channel conv", expect_mode=2)


def test_spec_step_in_one_launch_graph_replay():
    """The one-launch speculative step captured once and replayed with new
    live counts written into its device buffer: each replay's windows
    equal the oracle's, and the conv's output does not depend on them."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    case = workloads.spec_decode()
    gc = workloads.spec_gather(case, real_count=0)
    x = case.x.to(DEV)
    w = case.weight.to(DEV)
    cache0 = case.cache.to(DEV)
    cache = cache0.clone()
    pos, bt, sm = case.positions.to(DEV), case.block_table.to(DEV), case.slot_mapping.to(DEV)
    qsl = case.query_start_loc.to(DEV)
    out = torch.full_like(x, SENTINEL)
    src = x.view(1, case.T, case.C)
    gpos = gc.abs_positions.to(DEV)
    rc = torch.zeros(1, dtype=torch.int32, device=DEV)
    gout = gc.out_init.to(DEV).clone()

    def step():
        lib.sconv_fused_insert_conv_gather([x], [w], cache, pos, bt, sm, [0], [case.ws],
                                           case.block_size, src, gpos, rc, gout, 3,
                                           activation="silu", use_residual=True,
                                           query_start_loc=qsl, num_reqs=case.num_reqs,
                                           outs=[out])
    lib.sconv_init()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    cc, btc, smc = case.compact()
    out_r, _, _, _ = oracle_fused(case, cache=cc, block_table=btc, slot_mapping=smc)
    live = live_rows(case)
    g = torch.Generator().manual_seed(98)
    for n in [0, 512, 7] + [int(v) for v in torch.randint(0, 513, (3,), generator=g)]:
        cache.copy_(cache0)
        out.fill_(SENTINEL)
        gout.copy_(gc.out_init.to(DEV))
        rc.fill_(n)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_close(to_np(out), out_r, "bf16", f"replay n={n} out", mask=live)
        g_r = oracle.gather_conv_window(to_np(gc.src), to_np(gc.abs_positions), n,
                                        to_np(gc.out_init), 3)
        assert_bits_equal(to_np(gout), g_r, f"replay n={n} windows")
        say(f"  replay n={n} ok")


# ------------------------------------------------------------------ SSM-state row gather

SSM_GATHER = [
    # name, dtype, num_chunks, state shape, max_count
    ("f32-vec", torch.float32, 11, (3, 4, 8), 23),        # 384-byte rows: 16-byte path
    ("bf16-vec", torch.bfloat16, 7, (2, 64, 16), 9),      # 4 KiB rows
    ("bf16-elem", torch.bfloat16, 5, (3, 15), 13),        # 90-byte rows: element path
    ("f32-big", torch.float32, 6, (16, 64, 256), 5),      # 1 MiB rows, many column blocks
]


def test_config_ssm_state_gather():
    """The benchmarked extraction at full size: 128 chunk states of 2 MiB
    (64 x 64 x 128 fp32), 128 slots at distinct indices, 96 live; the whole
    output bit for bit (dead slots keep their sentinel)."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(13)
    nc, shape, mc, live = 128, (64, 64, 128), 128, 96
    states = torch.randn((nc,) + shape, generator=g)
    idx = torch.randperm(nc, generator=g)
    out0 = torch.full((mc,) + shape, SENTINEL)
    say("ssm gather at full size: 128 x 2 MiB rows, 96 live")
    out_r = oracle.gather_ssm_state(to_np(states), to_np(idx), live, to_np(out0))
    out_g = out0.to(DEV)
    lib.gather_intermediate_ssm_state(states.to(DEV), idx.to(DEV),
                                      torch.tensor([live], dtype=torch.int32, device=DEV), out_g)
    assert_bits_equal(to_np(out_g), out_r, "full-size SSM-state gather")


@pytest.mark.parametrize("spec", SSM_GATHER, ids=[s[0] for s in SSM_GATHER])
def test_ssm_state_gather_sweep(spec):
    import depthwise_causal_conv1d_amd as lib
    import oracle
    name, dt, nc, shape, mc = spec
    g = torch.Generator().manual_seed(nc * 31 + mc)
    states = torch.randn((nc,) + shape, generator=g).to(dt)
    idx = torch.randint(0, nc, (mc,), generator=g)
    out0 = torch.full((mc,) + shape, SENTINEL).to(dt)
    say(f"ssm gather {name}: {nc} rows of {shape}, max_count {mc}")
    st_d, idx_d = states.to(DEV), idx.to(DEV)
    for n in (0, 1, mc // 2, mc, mc + 5, -2):
        out_r = oracle.gather_ssm_state(to_np(states), to_np(idx), n, to_np(out0))
        out_g = out0.to(DEV).clone()
        lib.gather_intermediate_ssm_state(st_d, idx_d,
                                          torch.tensor([n], dtype=torch.int32, device=DEV), out_g)
        assert_bits_equal(to_np(out_g), out_r, f"{name} n={n}")


def test_ssm_state_gather_graph_replay_with_device_count():
    """Grid fixed at capture (max_count); the live count and the indices
    change between replays through their fixed device buffers only."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(5)
    nc, shape, mc = 8, (4, 32, 16), 40
    states = torch.randn((nc,) + shape, generator=g)
    out0 = torch.full((mc,) + shape, SENTINEL)
    st_d = states.to(DEV)
    idx_d = torch.zeros(mc, dtype=torch.int64, device=DEV)
    rc = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = out0.to(DEV).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.gather_intermediate_ssm_state(st_d, idx_d, rc, out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.gather_intermediate_ssm_state(st_d, idx_d, rc, out)
    torch.cuda.synchronize()
    for n in (0, mc, 3, 17, 1):
        idx = torch.randint(0, nc, (mc,), generator=g)
        idx_d.copy_(idx.to(DEV))
        out.copy_(out0.to(DEV))
        rc.fill_(n)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_r = oracle.gather_ssm_state(to_np(states), to_np(idx), n, to_np(out0))
        assert_bits_equal(to_np(out), out_r, f"replay n={n}")


# ------------------------------------------------------------------ multi-token / ring update

UPD_TOKENS = [
    # name, dtype, W, state_len, seqlen, ring, layout, in_place, bias, indices
    ("bf16-w4-shift-1", torch.bfloat16, 4, 3, 1, False, "bdt", True, True, True),
    ("bf16-w4-ring-1", torch.bfloat16, 4, 3, 1, True, "bdt", False, True, True),
    ("bf16-w4-shift-4", torch.bfloat16, 4, 3, 4, False, "btd", True, True, True),
    ("bf16-w4-ring-7-L5", torch.bfloat16, 4, 5, 7, True, "btd", False, False, True),
    ("f32-w3-ring-4-L8", torch.float32, 3, 8, 4, True, "bdt", True, True, False),
    ("f32-w2-shift-7-L6", torch.float32, 2, 6, 7, False, "bdt", False, True, True),
    ("bf16-w1-shift-3", torch.bfloat16, 1, 0, 3, False, "btd", False, True, True),
    ("f32-w4-ring-9-L4", torch.float32, 4, 4, 9, True, "btd", True, False, True),
]


# Cases of the vector-lane kernel: state_len = W-1, channels contiguous
# ("btd"), dim a multiple of the lane width.  Dims 40 and 64 put several
# rows, with their own ring rotations, in one wave; dim 1024 spreads a row
# over several waves.  Seqlens 5 and 9 span several 4-token chunks.
UPD_TOKENS_VEC = [
    # name, dtype, W, state_len, seqlen, ring, layout, in_place, bias, indices, dim
    ("vec-bf16-w4-ring-4", torch.bfloat16, 4, 3, 4, True, "btd", False, True, True, 64),
    ("vec-bf16-w4-shift-5", torch.bfloat16, 4, 3, 5, False, "btd", True, True, False, 64),
    ("vec-bf16-w3-ring-9", torch.bfloat16, 3, 2, 9, True, "btd", False, False, True, 128),
    ("vec-bf16-w2-ring-1", torch.bfloat16, 2, 1, 1, True, "btd", True, True, True, 64),
    ("vec-f32-w4-ring-3", torch.float32, 4, 3, 3, True, "btd", False, True, True, 40),
    ("vec-f32-w2-shift-8", torch.float32, 2, 1, 8, False, "btd", False, True, True, 40),
    ("vec-bf16-w4-ring-1-wide", torch.bfloat16, 4, 3, 1, True, "btd", False, True, True, 1024),
    # ring positions without state indices (the index load reads a stand-in)
    ("vec-bf16-w4-ring-3-noidx", torch.bfloat16, 4, 3, 3, True, "btd", False, True, False, 64),
]


@pytest.mark.parametrize("spec", UPD_TOKENS, ids=[s[0] for s in UPD_TOKENS])
def test_update_tokens_sweep(spec):
    check_update_tokens(*spec, dim=40)


@pytest.mark.parametrize("spec", UPD_TOKENS_VEC, ids=[s[0] for s in UPD_TOKENS_VEC])
def test_update_tokens_vec_sweep(spec):
    check_update_tokens(*spec)


def check_update_tokens(name, dt, W, L, T, ring, layout, in_place, has_bias, has_idx, dim):
    """One multi-token update against the oracle: outputs (PAD rows
    untouched) and the whole state pool, bit for bit.  x and out share the
    layout: "bdt" (tokens contiguous) or "btd" (channels contiguous)."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()) % 1000)
    batch, slots = 7, 12
    xs = torch.randn(batch, dim, T, generator=g).to(dt)
    if layout == "btd":  # tokens outer, channels contiguous
        x = xs.permute(0, 2, 1).contiguous().permute(0, 2, 1)
    else:
        x = xs.contiguous()
    w = (torch.randn(dim, W, generator=g) * 0.5).to(dt)
    bias = (torch.randn(dim, generator=g) * 0.1).to(dt) if has_bias else None
    st = torch.full((slots, dim, max(L, 1)), float("nan")).to(dt)[:, :, :L]
    idx = torch.randperm(slots, generator=g)[:batch].to(torch.int32) if has_idx else None
    if idx is not None:
        idx[3] = -1  # PAD row
    live_slots = idx[idx >= 0].long() if idx is not None else torch.arange(batch)
    st[live_slots] = torch.randn(live_slots.numel(), dim, L, generator=g).to(dt)
    seqlens = torch.randint(0, 20, (batch,), generator=g).to(torch.int32) if ring else None
    if ring:
        seqlens[0] = 0
        seqlens[1] = 1
        seqlens[2] = 2
    say(f"update_tokens {name}: batch {batch} dim {dim} W {W} state_len {L} seqlen {T}")
    out0 = torch.full_like(xs, SENTINEL)
    out_r, st_r = oracle.causal_conv1d_update_tokens(
        to_np(xs), to_np(st), to_np(w), None if bias is None else to_np(bias), "silu",
        None if seqlens is None else to_np(seqlens), None if idx is None else to_np(idx), -1,
        out_init=to_np(xs if in_place else out0))
    def on_dev(t):  # same values, in this case's layout
        t = t.to(DEV)
        return t.contiguous() if layout == "bdt" else t.permute(0, 2, 1).contiguous().permute(0, 2, 1)
    xg = on_dev(x)
    stg = st.to(DEV)
    outg = None if in_place else on_dev(out0)
    res = lib.causal_conv1d_update_tokens(
        xg, stg, w.to(DEV), None if bias is None else bias.to(DEV), True,
        None if seqlens is None else seqlens.to(DEV), None if idx is None else idx.to(DEV), -1,
        out=outg)
    live = np.ones(batch, bool) if idx is None else to_np(idx) >= 0
    got = to_np(res)
    assert_close(got[live], out_r[live], dtype_name(dt), f"{name} out")
    assert_bits_equal(got[~live], out_r[~live], f"{name} PAD rows untouched")
    assert_bits_equal(to_np(stg), st_r, f"{name} state pool")
    assert_finite(to_np(stg)[live_slots.numpy()], f"{name} live states")


def test_config_ssm_spec_decode():
    """The benchmarked speculative step at full size: 8 rows x 4 draft tokens
    x 8192 channels, channels contiguous (the vector-lane kernel), ring
    states of W-1 columns in a 1024-slot pool at positions uniform in
    [0, 4096); three steps in a row, each checked against the oracle (out,
    and the whole pool bit for bit)."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(12)
    B, T, dim, W, slots = 8, 4, 8192, 4, 1024
    w = (torch.randn(dim, W, generator=g) * 0.5).to(torch.bfloat16)
    bias = (torch.randn(dim, generator=g) * 0.1).to(torch.bfloat16)
    pool = torch.randn(slots, dim, W - 1, generator=g).to(torch.bfloat16)
    ci = torch.randperm(slots, generator=g)[:B].to(torch.int32)
    pool_g, w_g, b_g, ci_g = pool.to(DEV), w.to(DEV), bias.to(DEV), ci.to(DEV)
    pool_r = to_np(pool)
    for step in range(3):
        x = torch.randn(B, T, dim, generator=g).to(torch.bfloat16)  # tokens outer
        seqlens = torch.randint(0, 4096, (B,), generator=g).to(torch.int32)
        say(f"ssm spec decode step {step}")
        out_r, pool_r = oracle.causal_conv1d_update_tokens(
            to_np(x.permute(0, 2, 1).contiguous()), pool_r, to_np(w), to_np(bias), "silu",
            to_np(seqlens), to_np(ci), -1)
        out_g = torch.empty(B, T, dim, dtype=torch.bfloat16, device=DEV)
        lib.causal_conv1d_update_tokens(x.to(DEV).permute(0, 2, 1), pool_g, w_g, b_g, True,
                                        seqlens.to(DEV), ci_g, -1, out=out_g.permute(0, 2, 1))
        assert_close(to_np(out_g.permute(0, 2, 1).contiguous()), out_r, "bf16", f"step {step} out")
        assert_bits_equal(to_np(pool_g), pool_r, f"step {step} pool")
        assert_finite(to_np(pool_g)[to_np(ci)], f"step {step} live states")


def test_update_ring_form_equals_tokens_entry():
    """causal_conv1d_update with cache_seqlens is the one-token ring update."""
    import depthwise_causal_conv1d_amd as lib
    import oracle
    g = torch.Generator().manual_seed(17)
    batch, dim, W = 9, 64, 4
    x = torch.randn(batch, dim, generator=g).to(torch.bfloat16)
    w = (torch.randn(dim, W, generator=g) * 0.5).to(torch.bfloat16)
    bias = (torch.randn(dim, generator=g) * 0.1).to(torch.bfloat16)
    st = torch.randn(batch, dim, W - 1, generator=g).to(torch.bfloat16)
    seqlens = torch.randint(0, 9, (batch,), generator=g).to(torch.int32)
    out_r, st_r = oracle.causal_conv1d_update_tokens(to_np(x)[:, :, None], to_np(st), to_np(w),
                                                     to_np(bias), "silu", to_np(seqlens), None, -1)
    stg = st.to(DEV)
    out = lib.causal_conv1d_update(x.to(DEV), stg, w.to(DEV), bias.to(DEV), True,
                                   seqlens.to(DEV), None, -1, out=torch.empty_like(x, device=DEV))
    assert_close(to_np(out), out_r[:, :, 0], "bf16", "ring update out")
    assert_bits_equal(to_np(stg), st_r, "ring update state")
    assert_finite(to_np(stg), "ring update state")


# ------------------------------------------------------------------ random SSM-side sweep

def _ssm_rng(op, k):
    return np.random.default_rng(zlib.crc32(f"{op}-{k}".encode()))


@pytest.mark.parametrize("k", range(12))
def test_varlen_random_sweep(k):
    """Seeded random varlen launches: lengths including 0 and 1, vector and
    odd dims, W 1-4, some sequences with a state, PAD sequences, padded x
    rows, bias and activation drawn at random; out-of-place and in place."""
    rng = _ssm_rng("varlen", k)
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    lane = 8 if dt == torch.bfloat16 else 4
    n = int(rng.integers(1, 7))
    lens = [int(v) for v in rng.choice([0, 1, 2, 3, 17, 64, 255, 513, 1000], n)]
    dim = lane * int(rng.integers(1, 6)) if rng.random() < 0.6 else int(rng.integers(1, 40))
    W = int(rng.integers(1, 5))
    spec = (f"random-varlen-{k}", dt, lens, dim, W, int(rng.integers(0, n + 1)),
            int(rng.integers(0, n // 2 + 1)), None if rng.random() < 0.3 else 0.1,
            "silu" if rng.random() < 0.7 else None, int(rng.choice([0, 0, 5])))
    test_varlen_sweep(spec)


@pytest.mark.parametrize("k", range(12))
def test_update_tokens_random_sweep(k):
    """Seeded random multi-token updates: seqlen 1-9, state length W-1..8,
    shift or ring states, both x layouts, vector or odd dims, in place or
    not, with and without bias and indices."""
    rng = _ssm_rng("update_tokens", k)
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    W = int(rng.integers(1, 5))
    L = W - 1 if rng.random() < 0.5 else int(rng.integers(W - 1, 9))
    ring = bool(L >= 1 and rng.random() < 0.6)
    dim = 2 * int(rng.integers(1, 40)) if rng.random() < 0.7 else 2 * int(rng.integers(1, 20)) + 1
    check_update_tokens(f"random-update-tokens-{k}", dt, W, L, int(rng.integers(1, 10)), ring,
                        "btd" if rng.random() < 0.6 else "bdt", bool(rng.random() < 0.4),
                        bool(rng.random() < 0.7), bool(rng.random() < 0.7), dim)


@pytest.mark.parametrize("k", range(8))
def test_update_random_sweep(k):
    """Seeded random one-token updates: W 1-4, vector or odd dims, with or
    without indices (one PAD row), in place or not."""
    rng = _ssm_rng("update", k)
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    dim = 2 * int(rng.integers(1, 100)) if rng.random() < 0.7 else 2 * int(rng.integers(1, 50)) + 1
    test_update_sweep(dt, int(rng.integers(1, 5)), dim, bool(rng.random() < 0.7),
                      bool(rng.random() < 0.4))


@pytest.mark.parametrize("k", range(8))
def test_gather_random_sweep(k):
    """Seeded random conv-window gathers: odd or vector channel counts,
    d_conv 1-4, short and long sources, live counts 0, some and all."""
    rng = _ssm_rng("gather", k)
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    lane = 8 if dt == torch.bfloat16 else 4
    conv_dim = lane * int(rng.integers(1, 70)) if rng.random() < 0.6 else int(rng.integers(1, 90))
    test_gather_sweep(dt, conv_dim, int(rng.integers(1, 5)), int(rng.integers(1, 300)))
