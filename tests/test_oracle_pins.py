"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties one oracle function to a textbook identity, a library
routine, brute force on tiny inputs, or an invariant the pages state, so that
a plausible mistake in the oracle (a dropped tap, a reversed weight, an
off-by-one in the same-forward test, a wrong head stride, a stray write)
fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from tests.helpers import as_float, assert_bits_equal, bits, to_np

pytestmark = pytest.mark.usefixtures("oracle_lib")


def orc():
    import oracle
    return oracle


def silu_np(v):
    return v / (1.0 + np.exp(-v))


# ------------------------------------------------------------------ scalars

def test_round_bf16_matches_library_rne_on_float32_values():
    """Round-to-nearest-even of float32 values against torch's conversion,
    including exact ties, the largest finite values and subnormals."""
    o = orc()
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    ties = (u & 0xFFFF0000) | 0x8000          # exactly halfway cases
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x00008000,
                        0x00018000, 0x807FFFFF, 0x3F808000, 0x3F818000], dtype=np.uint32)
    allu = np.concatenate([u, ties, special])
    f = allu.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([o.round_bf16(float(v)) for v in f], dtype=np.uint16)
    assert_bits_equal(got, want, "round_bf16")


def test_round_bf16_single_rounding_from_double():
    """Doubles just off a float32 tie must round by their true distance
    (a float32 detour would land on the tie and go to even instead)."""
    o = orc()
    for base_bits in (0x3F80, 0x4000, 0xC2C8, 0x0100):
        lo = o.bf16_to_float(base_bits)
        hi = o.bf16_to_float(base_bits + 1)
        mid = (lo + hi) / 2
        eps = abs(hi - lo) * 2.0**-30       # below float32 resolution of mid
        assert o.round_bf16(mid + math.copysign(eps, hi - lo)) == base_bits + 1
        assert o.round_bf16(mid - math.copysign(eps, hi - lo)) == base_bits
    assert o.round_bf16(float("inf")) == 0x7F80
    assert o.round_bf16(3.5e38) == 0x7F80
    assert o.round_bf16(-0.0) == 0x8000


def test_silu_closed_forms():
    o = orc()
    assert o.silu(0.0) == 0.0
    assert o.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert o.silu(60.0) == pytest.approx(60.0, rel=1e-15)
    assert abs(o.silu(-60.0)) < 1e-24
    for v in np.linspace(-12, 12, 97):
        # sigma(v) + sigma(-v) = 1  =>  silu(v) - silu(-v) = v
        assert o.silu(v) - o.silu(-v) == pytest.approx(v, abs=1e-13)


# ------------------------------------------------------------------ metadata

@pytest.mark.parametrize("seed", range(6))
def test_metadata_matches_searchsorted(seed):
    """seq_idx is the sorted-search position of each row among the request
    starts (empty requests skipped, overflow clamped), query_start its start,
    padded rows zero."""
    o = orc()
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 40))
    lens = rng.integers(0, 9, R)
    lens[rng.random(R) < 0.3] = 0                   # empty requests
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(qsl[-1])
    num_actual = total + int(rng.integers(0, 3))     # rows past the last request clamp
    num_padded = num_actual + int(rng.integers(0, 20))
    si, qs = o.seq_metadata(qsl, R, num_actual, num_padded)
    t = np.arange(num_actual)
    want = np.searchsorted(qsl[1:R], t, side="right").astype(np.int32)
    np.testing.assert_array_equal(si[:num_actual], want)
    np.testing.assert_array_equal(qs[:num_actual], qsl[want])
    assert (si[num_actual:] == 0).all() and (qs[num_actual:] == 0).all()
    # every non-empty request's rows map back to it
    for r in range(R):
        assert (si[qsl[r]:qsl[r + 1]] == r).all()


def test_metadata_argument_errors():
    o = orc()
    qsl = np.array([0, 3], np.int32)
    with pytest.raises(ValueError):
        o.seq_metadata(qsl, 1, 3, 2)
    si, qs = o.seq_metadata(qsl, 1, 0, 5)
    assert (si == 0).all() and (qs == 0).all()


# ------------------------------------------------------------------ fused insert + conv

def _call_fused(case, seq_idx=None, query_start=None, out_init=None, slot_mapping=None):
    o = orc()
    if seq_idx is None:
        seq_idx, query_start = o.seq_metadata(to_np(case.query_start_loc), case.num_reqs,
                                              case.num_actual, case.T)
    return o.fused_insert_conv(
        to_np(case.x), to_np(case.weight), to_np(case.cache), to_np(case.positions),
        to_np(case.block_table), seq_idx, to_np(case.slot_mapping) if slot_mapping is None else slot_mapping,
        query_start, case.off_s, case.ws, case.block_size, case.activation, case.use_residual,
        out_init=out_init)


def test_fused_w1_identity_and_scale():
    """W=1: out = act(w*x) + x; with w=1, no activation and no residual the
    op is the identity, bit for bit, in every element type."""
    o = orc()
    for dt in (torch.float64, torch.float32, torch.bfloat16):
        case = workloads.fused_case(5, [7, 3], [20, 0], H=3, D=16, ws=4, off_s=8, block_size=8,
                                    W=1, dtype=dt, activation=None, use_residual=False)
        case.weight = torch.ones_like(case.weight)
        out, _ = _call_fused(case)
        assert_bits_equal(out, to_np(case.x), f"identity {dt}")
    case = workloads.fused_case(6, [9, 4], [3, 11], H=2, D=8, ws=4, off_s=4, block_size=4,
                                W=1, dtype=torch.float64, activation="silu", use_residual=True)
    out, _ = _call_fused(case)
    x, w = to_np(case.x), to_np(case.weight)[:, 0]
    np.testing.assert_allclose(out, silu_np(w * x) + x, rtol=1e-14, atol=0)


@pytest.mark.parametrize("act,res", [(None, False), ("silu", True), ("silu", False)])
def test_fused_zero_history_equals_torch_conv1d(act, res):
    """Requests starting at position 0: each is a zero-padded causal
    depthwise conv, i.e. torch conv1d with W-1 left padding and groups=C."""
    lens = [37, 1, 64, 5]
    case = workloads.fused_case(11, lens, [0] * 4, H=4, D=24, ws=6, off_s=12, block_size=16,
                                W=4, dtype=torch.float64, activation=act, use_residual=res)
    out, _ = _call_fused(case)
    x = case.x
    w = case.weight
    qsl = case.query_start_loc.tolist()
    for r in range(len(lens)):
        xr = x[qsl[r]:qsl[r + 1]]
        L = xr.shape[0]
        y = F.conv1d(xr.T[None], w[:, None, :], padding=3, groups=case.C)[0, :, :L].T
        if act:
            y = F.silu(y)
        if res:
            y = y + xr
        np.testing.assert_allclose(out[qsl[r]:qsl[r + 1]], y.numpy(), rtol=1e-12, atol=1e-14)


def _materialized_reference(case):
    """Brute force with a different structure: rebuild each request's whole
    input sequence (cache history + new rows) by position, then convolve it."""
    x = as_float(to_np(case.x))
    w = as_float(to_np(case.weight))
    cache = as_float(to_np(case.cache))
    bt = to_np(case.block_table)
    N, W, H, ws, off = case.block_size, case.W, case.H, case.ws, case.off_s
    qsl = case.query_start_loc.tolist()
    pos = case.positions.tolist()
    out = {}
    for r in range(case.num_reqs):
        rows = range(qsl[r], qsl[r + 1])
        if not len(rows):
            continue
        first = pos[rows[0]]
        seq = {}
        for p in range(max(0, first - (W - 1)), first):
            blk = bt[r, p // N]
            seq[p] = np.concatenate([cache[blk, h, p % N, off:off + ws] for h in range(H)])
        for t in rows:
            seq[pos[t]] = x[t]
        for t in rows:
            acc = np.zeros(case.C)
            for k in range(W):
                p = pos[t] - (W - 1) + k
                acc = acc + w[:, k] * (seq[p] if p >= 0 else 0.0)
            y = silu_np(acc) if case.activation else acc
            if case.use_residual:
                y = y + x[t]
            out[t] = y
    return out


@pytest.mark.parametrize("seed", range(4))
def test_fused_brute_force_and_full_cache_diff(seed):
    """Against a materialized-sequence brute force, with history in the
    cache, several requests per tile, PAD rows and padded tail rows; the
    post-call cache equals the snapshot with exactly the non-PAD slots'
    stream sub-range replaced (full diff, so stray writes show)."""
    rng = np.random.default_rng(100 + seed)
    R = 5
    new = [int(v) for v in rng.integers(1, 12, R)]
    ctx = [int(v) for v in rng.integers(0, 40, R)]
    ctx[0] = 0
    ctx[1] = 2            # history shorter than W-1
    case = workloads.fused_case(seed, new, ctx, H=3, D=20, ws=4, off_s=8, block_size=4, W=4,
                                dtype=torch.float64, pad_count=3, tail_pad=4,
                                activation="silu" if seed % 2 else None,
                                use_residual=bool(seed % 3))
    sentinel = np.full((case.T, case.C), -12345.0)
    out, cache_after = _call_fused(case, out_init=sentinel)
    ref = _materialized_reference(case)
    sm = case.slot_mapping.tolist()
    for t in range(case.T):
        if sm[t] < 0:
            assert (out[t] == -12345.0).all(), f"PAD row {t} written"
        else:
            np.testing.assert_allclose(out[t], ref[t], rtol=1e-13, atol=0, err_msg=f"row {t}")
            assert np.isfinite(out[t]).all()     # poison never read
    expect = to_np(case.cache).copy()
    x = to_np(case.x)
    N = case.block_size
    for t in range(case.T):
        if sm[t] < 0:
            continue
        for h in range(case.H):
            expect[sm[t] // N, h, sm[t] % N, case.off_s:case.off_s + case.ws] = \
                x[t, h * case.ws:(h + 1) * case.ws]
    assert_bits_equal(cache_after, expect, "cache after insert")


def test_fused_pad_rows_do_not_change_other_outputs():
    """A PAD row is skipped (no output, no slot write) but its input is still
    a same-forward tap: every other row matches the call without PAD."""
    case = workloads.fused_case(21, [9, 6, 12], [5, 0, 30], H=2, D=8, ws=4, off_s=0,
                                block_size=4, W=4, dtype=torch.float64, pad_count=5)
    sm = to_np(case.slot_mapping).copy()
    out_pad, _ = _call_fused(case, out_init=np.full((case.T, case.C), 7.0))
    case_nopad = workloads.fused_case(21, [9, 6, 12], [5, 0, 30], H=2, D=8, ws=4, off_s=0,
                                      block_size=4, W=4, dtype=torch.float64, pad_count=0)
    out_full, _ = _call_fused(case_nopad)
    live = sm >= 0
    assert (~live).sum() == 5
    assert_bits_equal(out_pad[live], out_full[live], "non-PAD rows")
    assert (out_pad[~live] == 7.0).all()


@pytest.mark.parametrize("dt", [torch.float64, torch.bfloat16])
def test_fused_prefill_equals_stepwise_decode(dt):
    """One multi-token call equals feeding the same tokens one decode step
    at a time, each step reading the previous steps' writes from the cache:
    same outputs and same final cache, bit for bit."""
    o = orc()
    new = [6, 1, 9, 4]
    ctx = [0, 17, 2, 33]
    case = workloads.fused_case(31, new, ctx, H=2, D=12, ws=4, off_s=4, block_size=4, W=4,
                                dtype=dt, activation="silu", use_residual=True)
    out_all, cache_all = _call_fused(case)
    x = to_np(case.x)
    qsl = case.query_start_loc.tolist()
    cache = to_np(case.cache)
    out_step = np.zeros_like(out_all)
    for s in range(max(new)):
        rows = [qsl[r] + s for r in range(len(new)) if s < new[r]]
        reqs = [r for r in range(len(new)) if s < new[r]]
        out_s, cache = o.fused_insert_conv(
            x[rows], to_np(case.weight), cache, to_np(case.positions)[rows],
            to_np(case.block_table), np.array(reqs, np.int32),
            to_np(case.slot_mapping)[rows], np.arange(len(rows), dtype=np.int32),
            case.off_s, case.ws, case.block_size, "silu", True)
        out_step[rows] = out_s
    assert_bits_equal(out_step, out_all, "outputs")
    assert_bits_equal(cache, cache_all, "cache")


def test_fused_streams_touch_only_their_subrange():
    """Two streams of one cache (different off_s) commute and never write
    outside their own D sub-range."""
    c0 = workloads.fused_case(41, [5, 7], [3, 9], H=2, D=16, ws=4, off_s=0, block_size=4,
                              W=4, dtype=torch.float64)
    c1 = workloads.FusedCase(**{**c0.__dict__, "off_s": 8,
                                "x": torch.randn(c0.T, c0.C, dtype=torch.float64)})
    o = orc()
    si, qs = o.seq_metadata(to_np(c0.query_start_loc), c0.num_reqs, c0.num_actual, c0.T)
    args = lambda c, cache: (to_np(c.x), to_np(c.weight), cache, to_np(c.positions),
                             to_np(c.block_table), si, to_np(c.slot_mapping), qs,
                             c.off_s, c.ws, c.block_size, "silu", True)
    cache = to_np(c0.cache)
    a0, k = o.fused_insert_conv(*args(c0, cache))
    a1, k = o.fused_insert_conv(*args(c1, k))
    b1, k2 = o.fused_insert_conv(*args(c1, cache))
    b0, k2 = o.fused_insert_conv(*args(c0, k2))
    assert_bits_equal(k, k2, "cache")
    assert_bits_equal(a0, b0, "stream 0")
    assert_bits_equal(a1, b1, "stream 1")
    untouched = np.ones(16, bool)
    untouched[0:4] = untouched[8:12] = False
    assert_bits_equal(k[..., untouched], cache[..., untouched], "other sub-ranges")


def test_fused_streams_order_free_and_each_stream_alone():
    """Four streams of one layer (different widths, activations and residual
    flags, PAD rows): any order of application gives the same bits, every
    stream's output equals that stream run alone on the original cache, and
    columns outside every stream's range keep their bits."""
    cases = workloads.fused_streams_case(
        43, [6, 1, 9], [5, 0, 12], H=3, D=24, streams=[(0, 4), (4, 8), (16, 2), (20, 4)],
        block_size=4, W=4, dtype=torch.float64, pad_count=2,
        activations=["silu", None, "silu", None], residuals=[True, True, False, False])
    o = orc()
    c0 = cases[0]
    si, qs = o.seq_metadata(to_np(c0.query_start_loc), c0.num_reqs, c0.num_actual, c0.T)
    common = (to_np(c0.positions), to_np(c0.block_table), si, to_np(c0.slot_mapping), qs,
              c0.block_size)
    spec = lambda c: {"x": to_np(c.x), "weight": to_np(c.weight), "off_s": c.off_s,
                      "ws": c.ws, "activation": c.activation, "use_residual": c.use_residual}
    cache = to_np(c0.cache)
    outs, k = o.fused_insert_conv_streams([spec(c) for c in cases], cache, *common)
    routs, rk = o.fused_insert_conv_streams([spec(c) for c in cases[::-1]], cache, *common)
    assert_bits_equal(k, rk, "cache, reversed order")
    for i, c in enumerate(cases):
        assert_bits_equal(outs[i], routs[len(cases) - 1 - i], f"stream {i}, reversed order")
        alone, _ = o.fused_insert_conv(spec(c)["x"], spec(c)["weight"], cache, *common[:5],
                                       c.off_s, c.ws, c.block_size, c.activation,
                                       c.use_residual)
        assert_bits_equal(outs[i], alone, f"stream {i} alone")
    untouched = np.ones(24, bool)
    for c in cases:
        untouched[c.off_s:c.off_s + c.ws] = False
    assert untouched.sum() == 6
    assert_bits_equal(k[..., untouched], cache[..., untouched], "columns of no stream")


def test_fused_rejects_out_of_table_reads():
    case = workloads.fused_case(3, [2], [40], H=1, D=4, ws=4, block_size=4, W=4,
                                dtype=torch.float64)
    o = orc()
    si, qs = o.seq_metadata(to_np(case.query_start_loc), 1, case.T, case.T)
    with pytest.raises(ValueError):
        o.fused_insert_conv(to_np(case.x), to_np(case.weight), to_np(case.cache),
                            to_np(case.positions), to_np(case.block_table)[:, :3], si,
                            to_np(case.slot_mapping), qs, 0, 4, 4, None, True)


# ------------------------------------------------------------------ SSM-style ops

def _varlen(case, out_init=None, x=None):
    o = orc()
    return o.causal_conv1d_varlen_fwd(
        to_np(case.x) if x is None else x, to_np(case.weight),
        None if case.bias is None else to_np(case.bias), to_np(case.conv_states),
        to_np(case.query_start_loc), to_np(case.cache_indices),
        to_np(case.has_initial_state), case.activation, case.pad_slot_id, out_init=out_init)


def test_varlen_zero_state_equals_torch_conv1d_with_bias():
    case = workloads.varlen_case(51, [13, 1, 40, 2], dim=6, num_slots=9, W=4,
                                 dtype=torch.float64, init_count=0, bias_std=0.3)
    out, st = _varlen(case)
    x, w, b = case.x, case.weight, case.bias
    qsl = case.query_start_loc.tolist()
    ci = case.cache_indices.tolist()
    for s in range(4):
        xs = x[:, qsl[s]:qsl[s + 1]]
        L = xs.shape[1]
        y = F.silu(F.conv1d(xs[None], w[:, None, :], b, padding=3, groups=6)[0, :, :L])
        np.testing.assert_allclose(out[:, qsl[s]:qsl[s + 1]], y.numpy(), rtol=1e-12, atol=1e-14)
        # final state: the last W-1 logical inputs (zeros before the start)
        xp = np.concatenate([np.zeros((6, 3)), xs.numpy()], axis=1)
        assert_bits_equal(st[ci[s]], xp[:, -3:], "final state")


def test_varlen_initial_state_equals_fused_history():
    """An initial state s is the same as fused_insert_conv with s sitting in
    the cache at the W-1 positions before the sequence (residual off)."""
    o = orc()
    L, dim = 11, 8
    vc = workloads.varlen_case(61, [L], dim=dim, num_slots=3, W=4, dtype=torch.float64,
                               init_count=1, bias_std=None)
    out_v, _ = _varlen(vc)
    s = to_np(vc.conv_states)[int(vc.cache_indices[0])]          # [dim, 3]
    fc = workloads.fused_case(62, [L], [3], H=2, D=4, ws=4, off_s=0, block_size=4, W=4,
                              dtype=torch.float64, activation="silu", use_residual=False,
                              x=vc.x.T.contiguous(), weight=vc.weight)
    cache = to_np(fc.cache).copy()
    bt = to_np(fc.block_table)
    for p in range(3):
        for h in range(2):
            cache[bt[0, p // 4], h, p % 4, 0:4] = s[h * 4:(h + 1) * 4, p]
    si, qs = o.seq_metadata(to_np(fc.query_start_loc), 1, L, L)
    out_f, _ = o.fused_insert_conv(to_np(fc.x), to_np(fc.weight), cache, to_np(fc.positions),
                                   bt, si, to_np(fc.slot_mapping), qs, 0, 4, 4, "silu", False)
    assert_bits_equal(out_v.T, out_f, "varlen vs fused")


@pytest.mark.parametrize("dt", [torch.float64, torch.bfloat16])
def test_varlen_prefill_then_updates_equals_longer_prefill(dt):
    """prefill(L) then k decode updates == prefill(L+k): same outputs and the
    same final states, bit for bit."""
    o = orc()
    L, k, dim = 9, 6, 5
    full = workloads.varlen_case(71, [L + k, 2], dim=dim, num_slots=4, W=4, dtype=dt,
                                 init_count=2)
    out_full, st_full = _varlen(full)
    x = to_np(full.x)
    ci = to_np(full.cache_indices)
    # prefill of the first L tokens of sequence 0 (sequence 1 unchanged)
    xp = np.concatenate([x[:, :L], x[:, L + k:]], axis=1)
    qsl = np.array([0, L, L + 2], np.int32)
    out_p, st = o.causal_conv1d_varlen_fwd(
        xp, to_np(full.weight), to_np(full.bias), to_np(full.conv_states), qsl, ci,
        to_np(full.has_initial_state), "silu", -1)
    outs = [out_p[:, :L]]
    for j in range(k):
        xs = np.ascontiguousarray(x[:, L + j][None, :])
        y, st = o.causal_conv1d_update(xs, st, to_np(full.weight), to_np(full.bias), "silu",
                                       ci[:1], -1)
        outs.append(y.T)
    assert_bits_equal(np.concatenate(outs, axis=1), out_full[:, :L + k], "outputs")
    assert_bits_equal(st, st_full, "states")


def test_update_from_zero_state_equals_causal_conv_and_shifts_state():
    o = orc()
    dim, steps = 7, 9
    xs = torch.randn(steps, dim, dtype=torch.float64, generator=torch.Generator().manual_seed(5))
    w = torch.randn(dim, 4, dtype=torch.float64, generator=torch.Generator().manual_seed(6))
    b = torch.randn(dim, dtype=torch.float64, generator=torch.Generator().manual_seed(7))
    st = np.zeros((2, dim, 3))
    outs = []
    for s in range(steps):
        y, st = o.causal_conv1d_update(xs[s:s + 1].numpy(), st, w.numpy(), b.numpy(), None,
                                       np.array([1], np.int32), -1)
        outs.append(y[0])
        hist = np.concatenate([np.zeros((3, dim)), xs[:s + 1].numpy()])[-3:].T
        assert_bits_equal(st[1], hist, f"state after step {s}")
        assert (st[0] == 0).all()
    ref = F.conv1d(xs.T[None], w[:, None, :], b, padding=3, groups=dim)[0, :, :steps].T
    np.testing.assert_allclose(np.array(outs), ref.numpy(), rtol=1e-12, atol=1e-14)


def test_ssm_w1_and_pad_sequences():
    """W=1 has an empty state: out = act(bias + w*x).  PAD sequences and PAD
    decode rows are left untouched."""
    o = orc()
    case = workloads.varlen_case(81, [4, 5, 3], dim=3, num_slots=5, W=1, dtype=torch.float64,
                                 pad_seqs=1, bias_std=0.2)
    out, st = _varlen(case, out_init=np.full((3, 12), 9.0))
    x, w, b = to_np(case.x), to_np(case.weight)[:, 0], to_np(case.bias)
    qsl = case.query_start_loc.tolist()
    for s, slot in enumerate(case.cache_indices.tolist()):
        seg = slice(qsl[s], qsl[s + 1])
        if slot == -1:
            assert (out[:, seg] == 9.0).all()
        else:
            np.testing.assert_allclose(out[:, seg], silu_np(b[:, None] + w[:, None] * x[:, seg]),
                                       rtol=1e-14)
    states = np.random.default_rng(0).standard_normal((4, 3, 3))
    xd = np.random.default_rng(1).standard_normal((3, 3))
    y, st2 = o.causal_conv1d_update(xd, states, np.ones((3, 4)), None, None,
                                    np.array([2, -1, 0], np.int32), -1,
                                    out_init=np.full((3, 3), 5.0))
    assert (y[1] == 5.0).all()
    assert_bits_equal(st2[1], states[1], "unused slot")
    assert_bits_equal(st2[3], states[3], "unused slot")
    np.testing.assert_allclose(y[0], states[2].sum(1) + xd[0], rtol=1e-14)


# ------------------------------------------------------------------ gather

@pytest.mark.parametrize("real_count", [0, 1, 17, 40, 41, 1000, -3])
def test_gather_matches_numpy_fancy_indexing(real_count):
    o = orc()
    rng = np.random.default_rng(real_count + 10)
    seq_len, cd, d, mc = 23, 6, 3, 40
    src = rng.standard_normal((seq_len, cd)).astype(np.float32)
    pos = rng.integers(-2, seq_len + 4, mc).astype(np.int32)
    out0 = np.full((mc, cd, d), -1.0, np.float32)
    got = o.gather_conv_window(src, pos, real_count, out0, d)
    n = min(max(real_count, 0), mc)
    rows = np.clip(pos[:, None] + np.arange(-d, 0)[None, :], 0, seq_len - 1)   # [mc, d]
    want = out0.copy()
    want[:n] = np.transpose(src[rows[:n]], (0, 2, 1))
    assert_bits_equal(got, want, "gather")


def test_gather_window_equals_prefill_final_state():
    """With d_conv = W-1, the window gathered at p equals the state a
    prefill of the first p rows leaves in its slot."""
    o = orc()
    seq_len, dim = 20, 5
    src = np.random.default_rng(3).standard_normal((seq_len, dim))
    w = np.ones((dim, 4))
    for p in range(3, seq_len + 1):
        _, st = o.causal_conv1d_varlen_fwd(np.ascontiguousarray(src[:p].T), w, None,
                                           np.zeros((1, dim, 3)), np.array([0, p], np.int32),
                                           np.array([0], np.int32), None, None, -1)
        g = o.gather_conv_window(src, np.array([p], np.int32), 1, np.zeros((1, dim, 3)), 3)
        assert_bits_equal(g[0], st[0], f"p={p}")


# ------------------------------------------------------------------ multi-token / ring update

def _upd_inputs(seed, batch, dim, W, L, seqlen, slots):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, dim, seqlen))
    w = rng.standard_normal((dim, W)) * 0.5
    bias = rng.standard_normal(dim) * 0.1
    st = rng.standard_normal((slots, dim, L))
    idx = rng.permutation(slots)[:batch].astype(np.int32)
    return x, w, bias, st, idx


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_update_tokens_one_token_equals_single_update(W):
    """seqlen 1 with a W-1 state is exactly causal_conv1d_update (f64 and
    bf16 bits), PAD rows included."""
    o = orc()
    x, w, bias, st, idx = _upd_inputs(W, 6, 5, W, W - 1, 1, 9)
    idx[2] = -1
    for cast in (lambda a: a, lambda a: to_np(torch.from_numpy(a).to(torch.bfloat16))):
        out_a, st_a = o.causal_conv1d_update(cast(np.ascontiguousarray(x[:, :, 0])), cast(st),
                                             cast(w), cast(bias), "silu", idx, -1)
        out_b, st_b = o.causal_conv1d_update_tokens(cast(x), cast(st), cast(w), cast(bias),
                                                    "silu", None, idx, -1)
        assert_bits_equal(out_b[:, :, 0], out_a, "out")
        assert_bits_equal(st_b, st_a, "state")


@pytest.mark.parametrize("L", [3, 5])
def test_update_tokens_equals_one_token_steps(L):
    """k tokens in one shift-state call equal k one-token calls, outputs and
    final state bit for bit (a state longer than W-1 keeps more history)."""
    o = orc()
    x, w, bias, st, idx = _upd_inputs(L, 4, 6, 4, L, 7, 5)
    out_m, st_m = o.causal_conv1d_update_tokens(x, st, w, bias, "silu", None, idx, -1)
    cur = st
    for i in range(7):
        oi, cur = o.causal_conv1d_update_tokens(np.ascontiguousarray(x[:, :, i:i + 1]), cur, w,
                                                bias, "silu", None, idx, -1)
        assert_bits_equal(out_m[:, :, i], oi[:, :, 0], f"token {i}")
    assert_bits_equal(st_m, cur, "state")


def test_update_tokens_ring_fresh_sequence_equals_zero_padded_conv():
    """A ring state fed from position 0 in calls of 3, 1, 5 and 2 tokens gives
    the zero-padded causal conv of all 11 inputs (torch conv1d, f64)."""
    o = orc()
    W, L, dim = 4, 5, 3
    rng = np.random.default_rng(12)
    xs = rng.standard_normal((1, dim, 11))
    w = rng.standard_normal((dim, W)) * 0.5
    bias = rng.standard_normal(dim) * 0.1
    st = np.zeros((1, dim, L))
    outs, s = [], 0
    for n in (3, 1, 5, 2):
        oi, st = o.causal_conv1d_update_tokens(np.ascontiguousarray(xs[:, :, s:s + n]), st, w,
                                               bias, "silu", np.array([s], np.int32), None, -1)
        outs.append(oi)
        s += n
    got = np.concatenate(outs, axis=2)
    ref = F.conv1d(F.pad(torch.from_numpy(xs), (W - 1, 0)), torch.from_numpy(w)[:, None, :],
                   torch.from_numpy(bias), groups=dim).numpy()
    np.testing.assert_allclose(got, silu_np(ref), rtol=1e-12, atol=1e-12)
    # the ring holds the last L inputs at their position's column
    for p in range(11 - L, 11):
        np.testing.assert_array_equal(st[0, :, p % L], xs[0, :, p])


def test_update_tokens_ring_equals_rotated_shift_state():
    """With s >= state_len, a ring call equals a shift call on the ring
    rotated into chronological order: same outputs, and the new ring is the
    new shift state rotated back (bit for bit)."""
    o = orc()
    W, L, T = 4, 6, 4
    x, w, bias, ring, idx = _upd_inputs(21, 3, 4, W, L, T, 3)
    s = np.array([9, 14, 6], np.int32)
    out_r, ring_new = o.causal_conv1d_update_tokens(x, ring, w, bias, None, s, idx, -1)
    chrono = np.empty_like(ring)
    for b in range(3):
        sl = idx[b]
        for m in range(L):
            chrono[sl, :, m] = ring[sl, :, (s[b] - L + m) % L]
    out_s, chrono_new = o.causal_conv1d_update_tokens(x, chrono, w, bias, None, None, idx, -1)
    assert_bits_equal(out_r, out_s, "outputs")
    for b in range(3):
        sl = idx[b]
        for m in range(L):
            assert_bits_equal(ring_new[sl, :, (s[b] + T - L + m) % L], chrono_new[sl, :, m],
                              f"row {b} column {m}")


def test_update_tokens_ring_never_reads_before_position_zero():
    """s = 2 < W-1: the ring column of position -1 holds NaN and is never
    read; the outputs are the zero-padded conv of the stored positions 0, 1
    and the new inputs.  A PAD row keeps its output and state bits."""
    o = orc()
    W, L, dim = 4, 3, 2
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, dim, 3))
    w = rng.standard_normal((dim, W)) * 0.5
    ring = np.full((2, dim, L), np.nan)
    prev = rng.standard_normal((dim, 2))
    ring[0, :, 0], ring[0, :, 1] = prev[:, 0], prev[:, 1]
    idx = np.array([0, -1], np.int32)
    out0 = np.full((2, dim, 3), 7.0)
    got, ring_new = o.causal_conv1d_update_tokens(x, ring, w, None, None,
                                                  np.array([2, 0], np.int32), idx, -1,
                                                  out_init=out0)
    seq = np.concatenate([prev, x[0]], axis=1)[None]
    ref = F.conv1d(F.pad(torch.from_numpy(seq), (W - 1, 0)), torch.from_numpy(w)[:, None, :],
                   groups=dim).numpy()[0, :, 2:]
    np.testing.assert_allclose(got[0], ref, rtol=1e-12, atol=1e-12)
    assert_bits_equal(got[1], out0[1], "PAD row output")
    assert_bits_equal(ring_new[1], ring[1], "PAD row state")


@pytest.mark.parametrize("real_count", [0, 1, 17, 40, 55, -3])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ssm_state_gather_matches_numpy_row_indexing(real_count, dt):
    """Slots below the clamped count receive their state row bit for bit;
    the others keep their bits."""
    o = orc()
    rng = np.random.default_rng(real_count + 77)
    nc, shape, mc = 9, (3, 4, 5), 40
    if dt == "f32":
        states = rng.standard_normal((nc,) + shape).astype(np.float32)
        out0 = np.full((mc,) + shape, -1.0, np.float32)
    else:
        states = rng.integers(0, 2**16, (nc,) + shape).astype(np.uint16)
        out0 = np.full((mc,) + shape, 0xBEEF, np.uint16)
    idx = rng.integers(0, nc, mc).astype(np.int64)
    got = o.gather_ssm_state(states, idx, real_count, out0)
    n = min(max(real_count, 0), mc)
    want = out0.copy()
    want[:n] = states[idx[:n]]
    assert_bits_equal(got, want, "ssm gather")


def test_ssm_state_gather_rejects_out_of_range_rows():
    o = orc()
    states = np.zeros((4, 6), np.float32)
    idx = np.array([0, 4, 1], np.int64)
    with pytest.raises(ValueError, match="num_chunks"):
        o.gather_ssm_state(states, idx, 2, np.zeros((3, 6), np.float32))
    o.gather_ssm_state(states, idx, 1, np.zeros((3, 6), np.float32))  # slot 1 is dead


def test_named_workloads_are_well_formed():
    """The generators' layout obeys the preconditions the op relies on:
    slots point at the row's own position, no slot is written twice, and no
    written slot is a pre-forward tap of the same call."""
    for case in (workloads.tiny_prefill(),
                 workloads.fused_case(9, [5, 30, 1], [0, 70, 3], H=2, D=8, ws=4,
                                      block_size=16, pad_count=4)):
        N = case.block_size
        sm = case.slot_mapping.tolist()
        live = [s for s in sm if s >= 0]
        assert len(live) == len(set(live))
        qsl = case.query_start_loc.tolist()
        for r in range(case.num_reqs):
            for t in range(qsl[r], qsl[r + 1]):
                p = int(case.positions[t])
                if sm[t] >= 0:
                    assert sm[t] == int(case.block_table[r, p // N]) * N + p % N
                first = int(case.positions[qsl[r]])
                for q in range(max(0, first - 3), first):
                    assert int(case.block_table[r, q // N]) * N + q % N not in live


# ------------------------------------------------------------------ threaded forms

@pytest.mark.parametrize("threads", [2, 3, 8])
def test_threaded_oracle_equals_single_threaded(threads):
    """The row-split fused op and the channel-split varlen op (used to time
    the oracle on every host core) give the single-threaded bits, outputs
    and cache or states, including ranges that cut a request in two."""
    o = orc()
    from tests.gpu_util import oracle_fused
    case = workloads.fused_case(91, [9, 1, 30, 4, 17], [0, 21, 5, 40, 3], H=4, D=64, ws=16,
                                off_s=16, block_size=16, W=4, dtype="bf16", pad_count=4,
                                tail_pad=3)
    out1, cache1, si, qs = oracle_fused(case)
    out_n, cache_n = o.fused_insert_conv(
        to_np(case.x), to_np(case.weight), to_np(case.cache), to_np(case.positions),
        to_np(case.block_table), si, to_np(case.slot_mapping), qs, case.off_s, case.ws,
        case.block_size, "silu", True, out_init=to_np(torch.full_like(case.x, -777.0)),
        threads=threads)
    assert_bits_equal(out_n, out1, "fused out")
    assert_bits_equal(cache_n, cache1, "fused cache")
    v = workloads.varlen_case(92, [13, 1, 0, 70, 2], dim=24, num_slots=9, W=4, dtype="bf16",
                              init_count=2, pad_seqs=1)
    args = (to_np(v.x), to_np(v.weight), to_np(v.bias), to_np(v.conv_states),
            to_np(v.query_start_loc), to_np(v.cache_indices), to_np(v.has_initial_state),
            "silu", -1)
    a_out, a_st = o.causal_conv1d_varlen_fwd(*args)
    b_out, b_st = o.causal_conv1d_varlen_fwd(*args, threads=threads)
    assert_bits_equal(b_out, a_out, "varlen out")
    assert_bits_equal(b_st, a_st, "varlen states")
