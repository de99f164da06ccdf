"""The C ABI library loads, exports every entry point the header declares,
and rejects bad host arguments before touching the GPU (CPU only: no call
here reaches a kernel launch)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sconv.h")


@pytest.fixture(scope="module")
def lib():
    from depthwise_causal_conv1d_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from depthwise_causal_conv1d_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_five_ops():
    names = set(declared_functions())
    assert {"sconv_seq_metadata", "sconv_fused_insert_conv", "causal_conv1d_varlen_fwd",
            "causal_conv1d_update", "gather_intermediate_conv_window",
            "sconv_last_error"} <= names


def test_every_declared_symbol_is_exported(lib):
    from depthwise_causal_conv1d_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.EXPORTS)


def test_version_and_clean_error(lib):
    assert b"gfx950" in lib.sconv_version()


NULL = None


def test_metadata_rejects_bad_scalars(lib):
    rc = lib.sconv_seq_metadata(NULL, 1, 10, 5, NULL, 10, NULL, 10, NULL)
    assert rc == 1 and b"is below num_actual_tokens" in lib.sconv_last_error()
    rc = lib.sconv_seq_metadata(NULL, 1, 4, 8, NULL, 7, NULL, 8, NULL)
    assert rc == 1 and b"seq_idx_out holds 7 entries, 8 rows" in lib.sconv_last_error()
    rc = lib.sconv_seq_metadata(NULL, 1, 4, 8, NULL, 8, NULL, 6, NULL)
    assert rc == 1 and b"query_start_out holds 6 entries, 8 rows" in lib.sconv_last_error()
    rc = lib.sconv_seq_metadata(NULL, 0, 4, 8, NULL, 8, NULL, 8, NULL)
    assert rc == 1
    # nothing to do is a success and launches nothing
    assert lib.sconv_seq_metadata(NULL, 0, 0, 0, NULL, 0, NULL, 0, NULL) == 0


def _fused(lib, **kw):
    a = dict(x=NULL, xrs=16, w=NULL, wsc=4, wsk=1, cache=NULL, nb=8, H=2, N=16, D=32,
             cs0=1024, cs1=512, cs2=32, pos=NULL, bt=NULL, btrs=4, mb=4, si=NULL, sm=NULL,
             qs=NULL, out=NULL, ors=16, T=64, off=0, ws=8, W=4, dt=0, act=1, res=1)
    a.update(kw)
    return lib.sconv_fused_insert_conv(*a.values(), NULL)


def test_fused_rejects_bad_scalars(lib):
    assert _fused(lib, W=5) == 1 and b"W=5" in lib.sconv_last_error()
    assert _fused(lib, W=0) == 1
    assert _fused(lib, off=28) == 1 and b"outside D" in lib.sconv_last_error()
    assert _fused(lib, dt=7) == 1
    assert _fused(lib, act=3) == 1
    assert _fused(lib, T=-1) == 1
    assert _fused(lib, xrs=8) == 1            # row stride < C
    assert _fused(lib, cs2=16) == 1           # D rows overlap
    assert _fused(lib, T=0) == 0              # empty batch: no-op
    assert _fused(lib) == 1 and b"NULL" in lib.sconv_last_error()
    buf = (ctypes.c_uint8 * 64)()
    p = ctypes.addressof(buf)
    # out == x is rejected before anything runs
    assert _fused(lib, x=p, w=p, cache=p + 4096 * 1024, pos=p, bt=p, si=p, sm=p, qs=p,
                  out=p) == 1
    assert b"overlaps" in lib.sconv_last_error()


def _fused_qsl(lib, **kw):
    a = dict(x=NULL, xrs=16, w=NULL, wsc=4, wsk=1, cache=NULL, nb=8, H=2, N=16, D=32,
             cs0=1024, cs1=512, cs2=32, pos=NULL, bt=NULL, btrs=4, mb=4, qsl=NULL, nreq=2,
             sm=NULL, out=NULL, ors=16, T=64, off=0, ws=8, W=4, dt=0, act=1, res=1)
    a.update(kw)
    return lib.sconv_fused_insert_conv_qsl(*a.values(), NULL)


def test_folded_entry_rejects_bad_scalars(lib):
    """sconv_fused_insert_conv_qsl: the request offsets are required with
    rows to process, num_reqs must be >= 1, and every check of the
    per-row entry applies as well.  No call reaches a launch."""
    assert _fused_qsl(lib) == 1 and b"query_start_loc" in lib.sconv_last_error()
    one = ctypes.c_int32(0)
    q = ctypes.addressof(one)
    assert _fused_qsl(lib, qsl=q, nreq=0) == 1     # NULL buffers are checked first
    buf = (ctypes.c_uint8 * 1024)()
    b = ctypes.addressof(buf)
    # stand-in addresses, never dereferenced: validation fails first
    dev = dict(x=b, w=b, cache=b + (1 << 20), pos=b, bt=b, sm=b, out=b + (1 << 21))
    assert _fused_qsl(lib, qsl=q, nreq=0, **dev) == 1
    assert b"num_reqs" in lib.sconv_last_error()
    assert _fused_qsl(lib, qsl=q, W=5) == 1 and b"W=5" in lib.sconv_last_error()
    assert _fused_qsl(lib, qsl=q, off=28) == 1
    assert _fused_qsl(lib, T=0) == 0             # empty batch: no-op, offsets not needed


def test_ssm_ops_reject_bad_scalars(lib):
    v = lib.causal_conv1d_varlen_fwd
    assert v(NULL, 1, 1, NULL, 4, 1, NULL, NULL, 1, 1, 1, 1, NULL, 1, NULL, NULL, NULL, 1, 1, 8,
             8, 5, 1, 1, -1, NULL) == 1
    assert v(NULL, 1, 1, NULL, 4, 1, NULL, NULL, 1, 1, 1, 1, NULL, 0, NULL, NULL, NULL, 1, 1, 8,
             8, 4, 1, 1, -1, NULL) == 0            # batch 0: no-op
    u = lib.causal_conv1d_update
    one = ctypes.c_int32(1)
    assert u(NULL, 8, NULL, 1, 24, 3, 1, NULL, 4, 1, NULL, ctypes.addressof(one), NULL, NULL, 8,
             1, 8, 4, 1, 1, -1, NULL) == 1          # ring form: NULL x is still rejected
    t = lib.causal_conv1d_update_tokens
    args = lambda sl, L, W=4, ring=None: (NULL, 64, 1, 8, sl, NULL, 4, L, 24, L, 1, NULL, W, 1,
                                          NULL, ring, NULL, NULL, 64, 1, 8, 2, 8, W, 1, 1, -1,
                                          NULL)
    assert t(*args(3, 2)) == 1                          # state_len < W-1
    assert b"shorter than W-1" in lib.sconv_last_error()
    assert t(*args(3, 9)) == 2                          # state_len above 8
    assert t(*args(3, 0, W=1, ring=ctypes.addressof(one))) == 1   # ring needs a column
    assert t(*args(0, 3)) == 0                          # seqlen 0: no-op
    assert t(*args(3, 3)) == 1                          # NULL pointers
    assert u(NULL, 8, NULL, 1, 24, 3, 1, NULL, 4, 1, NULL, NULL, NULL, NULL, 8, 1, 8, 9, 1, 1,
             -1, NULL) == 1
    g = lib.gather_intermediate_conv_window
    assert g(NULL, 10, 8, 8, 1, NULL, NULL, 4, NULL, 24, 5, 1, NULL) == 2   # d_conv 5
    assert g(NULL, 0, 8, 8, 1, NULL, NULL, 4, NULL, 24, 3, 1, NULL) == 1    # seq_len 0
    assert g(NULL, 10, 8, 8, 1, NULL, NULL, 0, NULL, 24, 3, 1, NULL) == 0   # no slots
    assert g(NULL, 10, 8, 8, 1, NULL, NULL, 65536, NULL, 24, 3, 1, NULL) == 2  # grid rows
    assert b"65535" in lib.sconv_last_error()


def test_streams_entry_rejects_bad_host_arguments(lib):
    """sconv_fused_insert_conv_streams: stream count, overlapping column
    ranges and the two per-row request forms are checked on the host.  Every
    call has T = 0 or fails validation, so none launches a kernel."""
    from depthwise_causal_conv1d_amd._lib import StreamT
    f = lib.sconv_fused_insert_conv_streams
    one = ctypes.c_int32(0)

    def streams(*ranges):
        arr = (StreamT * max(1, len(ranges)))()
        for i, (off, ws) in enumerate(ranges):
            arr[i] = StreamT(None, 4 * ws, None, 4, 1, None, 4 * ws, off, ws, 1, 1)
        return arr

    # H=4, N=16, D=16, cs=(1024, 256, 16); T = 0 unless noted.
    def call(arr, n, seq=NULL, qs=NULL, qsl=NULL, T=0):
        return f(arr, n, NULL, 8, 4, 16, 16, 1024, 256, 16, NULL, NULL, 4, 4, seq, qs, qsl, 1,
                 NULL, T, 4, 1, NULL)

    ok = streams((0, 4), (4, 4), (8, 8))
    assert call(ok, 3, qsl=ctypes.addressof(one)) == 0                  # valid, T = 0: no-op
    assert call(ok, 0, qsl=ctypes.addressof(one)) == 1                  # no stream
    assert call(streams((0, 4), (4, 4), (8, 4), (12, 2), (14, 2)), 5,
                qsl=ctypes.addressof(one)) == 1                          # five streams
    assert b"num_streams" in lib.sconv_last_error()
    assert call(streams((0, 8), (4, 8)), 2, qsl=ctypes.addressof(one)) == 1   # overlap
    assert b"share cache columns" in lib.sconv_last_error()
    assert call(streams((12, 8)), 1, qsl=ctypes.addressof(one)) == 1     # past D
    assert call(ok, 3) == 1                                              # no request form
    assert b"either" in lib.sconv_last_error()
    assert call(ok, 3, seq=ctypes.addressof(one), qs=ctypes.addressof(one),
                qsl=ctypes.addressof(one)) == 1                          # both forms
    assert call(ok, 3, seq=ctypes.addressof(one), qs=ctypes.addressof(one)) == 0


def test_ssm_gather_rejects_bad_host_arguments(lib):
    g = lib.gather_intermediate_ssm_state
    assert g(NULL, 0, 8, 8, NULL, NULL, 4, NULL, 8, 0, NULL) == 1        # no rows
    assert g(NULL, 4, 8, 7, NULL, NULL, 4, NULL, 8, 0, NULL) == 1        # stride < row
    assert g(NULL, 4, 8, 8, NULL, NULL, 65536, NULL, 8, 0, NULL) == 2    # grid rows
    assert b"65535" in lib.sconv_last_error()
    assert g(NULL, 4, 8, 8, NULL, NULL, 4, NULL, 8, 7, NULL) == 1        # dtype
    assert g(NULL, 4, 8, 8, NULL, NULL, 0, NULL, 8, 0, NULL) == 0        # no slots: no-op
    assert g(NULL, 4, 8, 8, NULL, NULL, 4, NULL, 8, 0, NULL) == 1        # NULL pointers


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding has no CPU fallback: a missing library is an import error."""
    from depthwise_causal_conv1d_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_binding_rejects_strided_block_table_entries():
    """The C ABI takes one row stride for block_table, so the binding refuses
    a view whose entries within a row are not contiguous (checked before
    anything touches a device)."""
    import torch

    import depthwise_causal_conv1d_amd as sc
    T, H, ws, N, D, W = 4, 2, 8, 4, 16, 4
    x = torch.zeros(T, H * ws)
    w = torch.zeros(H * ws, W)
    cache = torch.zeros(8, H, N, D)
    pos = torch.arange(T, dtype=torch.int64)
    sm = torch.arange(T, dtype=torch.int64)
    bt = torch.zeros(1, 8, dtype=torch.int32)[:, ::2]  # stride(1) == 2
    meta = torch.zeros(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="contiguous entries"):
        sc.sconv_fused_insert_conv(x, w, cache, pos, bt, meta, sm, meta, 0, ws, N)
    with pytest.raises(ValueError, match="contiguous entries"):
        sc.sconv_fused_insert_conv_qsl(x, w, cache, pos, bt, torch.tensor([0, T], dtype=torch.int32),
                                       1, sm, 0, ws, N)


_HOST_PATHS = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from depthwise_causal_conv1d_amd import _lib
from depthwise_causal_conv1d_amd._lib import StreamT
lib = _lib.load()
arena = (ctypes.c_uint8 * (64 << 20))()
base = (ctypes.addressof(arena) + 4095) & ~4095
nxt = [base]
def buf(nbytes):  # distinct, 4 KiB-aligned host regions: never dereferenced here
    p = nxt[0]; nxt[0] += (nbytes + 4095) & ~4095; return p
results = []
def expect(name, rc):
    results.append((name, rc))
for dt, es in ((0, 4), (1, 2)):
    for H, ws, D, T, R in ((4, 32, 128, 64, 64), (4, 32, 128, 64, 16), (4, 32, 128, 60, 17),
                           (2, 6, 16, 40, 3), (32, 128, 512, 20000, 16)):
        C = H * ws
        x, w, out = buf(T * C * es), buf(C * 4 * es), buf(T * C * es)
        cache = buf(64 * H * 16 * D * es)
        pos, sm, bt = buf(T * 8), buf(T * 8), buf(R * 300 * 4)
        si, qs, qsl = buf(T * 4), buf(T * 4), buf((R + 1) * 4)
        expect(f"fused dt{dt} T{T} R{R}", lib.sconv_fused_insert_conv(
            x, C, w, 4, 1, cache, 64, H, 16, D, H * 16 * D, 16 * D, D, pos, bt, 300, 300,
            si, sm, qs, out, C, T, 0, ws, 4, dt, 1, 1, None))
        expect(f"fused-qsl dt{dt} T{T} R{R}", lib.sconv_fused_insert_conv_qsl(
            x, C, w, 4, 1, cache, 64, H, 16, D, H * 16 * D, 16 * D, D, pos, bt, 300, 300,
            qsl, R, sm, out, C, T, 0, ws, 4, dt, 1, 1, None))
        if D >= 2 * ws:
            arr = (StreamT * 2)(StreamT(x, C, w, 4, 1, out, C, 0, ws, 1, 1),
                                StreamT(buf(T * C * es), C, buf(C * 4 * es), 4, 1,
                                        buf(T * C * es), C, ws, ws, 0, 0))
            for q in (qsl, None):
                expect(f"streams dt{dt} T{T} R{R} folded={q is not None}",
                       lib.sconv_fused_insert_conv_streams(
                           arr, 2, cache, 64, H, 16, D, H * 16 * D, 16 * D, D, pos, bt, 300, 300,
                           None if q else si, None if q else qs, q, R, sm, T, 4, dt, None))
        # conv + window gather over the conv's x, in one launch or two
        g = _lib.WindowGather(x, T, C, C, 1, buf(64 * 4), buf(4), 64, buf(64 * C * 3 * es),
                              C * 3, 3)
        arr1 = (StreamT * 1)(StreamT(x, C, w, 4, 1, out, C, 0, ws, 1, 1))
        expect(f"conv+gather dt{dt} T{T} R{R}", lib.sconv_fused_insert_conv_gather(
            arr1, 1, cache, 64, H, 16, D, H * 16 * D, 16 * D, D, pos, bt, 300, 300, None, None,
            qsl, R, sm, T, 4, dt, ctypes.byref(g), None))
    dim = 64
    xs, st = buf(dim * 4096 * es), buf(16 * dim * 3 * es)
    expect(f"varlen dt{dt}", lib.causal_conv1d_varlen_fwd(
        xs, 4096, 1, buf(dim * 4 * es), 4, 1, buf(dim * es), st, 16, dim * 3, 3, 1, buf(12), 2,
        buf(8), buf(2), buf(dim * 4096 * es), 4096, 1, dim, 4096, 4, dt, 1, -1, None))
    for ring in (None, buf(32)):
        expect(f"update dt{dt} ring={ring is not None}", lib.causal_conv1d_update(
            buf(8 * dim * es), dim, st, 16, dim * 3, 3, 1, buf(dim * 4 * es), 4, 1, buf(dim * es),
            ring, buf(32), buf(8 * dim * es), dim, 8, dim, 4, dt, 1, -1, None))
        expect(f"update_tokens dt{dt} ring={ring is not None}", lib.causal_conv1d_update_tokens(
            buf(8 * 4 * dim * es), 4 * dim, 1, dim, 4, st, 16, 3, dim * 3, 3, 1,
            buf(dim * 4 * es), 4, 1, buf(dim * es), ring, buf(32), buf(8 * 4 * dim * es), 4 * dim,
            1, dim, 8, dim, 4, dt, 1, -1, None))
    expect(f"gather window dt{dt}", lib.gather_intermediate_conv_window(
        buf(2048 * dim * es), 2048, dim, dim, 1, buf(512 * 4), buf(4), 512, buf(512 * dim * 3 * es),
        dim * 3, 3, dt, None))
    expect(f"gather state dt{dt}", lib.gather_intermediate_ssm_state(
        buf(8 * 4096 * es), 8, 4096, 4096, buf(8 * 16), buf(4), 16, buf(16 * 4096 * es), 4096, dt,
        None))
expect("metadata", lib.sconv_seq_metadata(buf(68), 16, 64, 64, buf(256), 64, buf(256), 64, None))
expect("init", lib.sconv_init())
for name, rc in results:
    print(name, rc)
'''


def test_host_paths_reach_the_launch(tmp_path):
    """Every entry point, with valid host arguments of several shapes
    (decode-, spec- and prefill-shaped fused launches, folded or not, one
    and two streams, both dtypes, ring and shift updates), runs its whole
    host-side set-up and returns SCONV_ERR_HIP from the launch only because
    no GPU is present.  Runs in a child process so that a host crash fails
    the test instead of the run; skipped where a GPU is visible, since the
    buffers are host memory standing in for device pointers."""
    import subprocess
    import sys

    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: these stand-in pointers must not reach a launch")
    r = subprocess.run([sys.executable, "-c", _HOST_PATHS, ROOT], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, f"host path crashed (exit {r.returncode}): {r.stderr[-2000:]}"
    lines = [l.rsplit(" ", 1) for l in r.stdout.strip().splitlines()]
    assert len(lines) >= 40
    bad = [(n, rc) for n, rc in lines if rc != "3"]
    assert not bad, f"expected the launch error (3) everywhere, got {bad}"


# A 16-byte-aligned stand-in address: the plan query never dereferences
# its pointers, so the buffers are placed at fixed offsets from it.
STAND_IN = 1 << 24


def _plan(lib, T, num_reqs, H=32, ws=32, D=128, N=16, max_blocks=257, folded=True, W=4,
          streams=1, dt=1, gather=None, bt_rs=None):
    """sconv_fused_plan on stand-in addresses (16-byte aligned, never
    dereferenced): returns (rc, plan)."""
    from depthwise_causal_conv1d_amd import _lib
    C = H * ws
    base = STAND_IN
    # x, out of each stream and the cache at distant stand-in addresses
    arr = (_lib.StreamT * streams)()
    for s in range(streams):
        arr[s] = _lib.StreamT(base + (s + 1) * (1 << 40), C, base, W, 1,
                              base + (s + 1) * (1 << 40) + (1 << 39), C, s * ws, ws, 1, 1)
    cache = base + (1 << 44)
    plan = _lib.FusedPlan()
    meta = (None, None, base, num_reqs) if folded else (base, base, None, 0)
    rc = lib.sconv_fused_plan(arr, streams, cache, 1 << 16, H, N, D, H * N * D, N * D, D, base,
                              base, max_blocks if bt_rs is None else bt_rs, max_blocks, *meta,
                              base, T, W, dt,
                              None if gather is None else ctypes.byref(gather),
                              ctypes.byref(plan))
    return rc, plan


def test_plan_guessed_one_row_tiles_read_inside_the_table(lib):
    """Guessed one-row tiles read block-table row t ahead in the kernel; the
    plan must give them at least one entry (an empty read-ahead would index
    the entry before the row) and never more than the row holds."""
    cases = []
    for T, R in [(256, 256), (48, 48), (200, 50), (64, 16), (120, 40), (8, 8), (4096, 4096),
                 (2048, 512), (9, 3)]:
        for mb in (1, 3, 100, 257, 4097):
            for H, ws in ((32, 32), (2, 8), (64, 64)):
                cases.append((T, R, mb, H, ws))
    seen_guess_row = 0
    for T, R, mb, H, ws in cases:
        rc, plan = _plan(lib, T, R, H=H, ws=ws, D=max(ws, 128), max_blocks=mb)
        assert rc == 0, lib.sconv_last_error()
        if plan.request_mode == 3 and plan.rows_per_tile == 1:
            seen_guess_row += 1
            assert 1 <= plan.bt_row_entries <= min(mb, 256), (T, R, mb, plan.bt_row_entries)
            if plan.rows_per_request > 1:
                assert plan.bt_row_entries == 1
        else:
            assert plan.bt_row_entries == 0, (T, R, mb)
    assert seen_guess_row > 20


def test_plan_guess_needs_a_32_bit_table_stride(lib):
    """The guessed forms take the block-table row stride as a 32-bit leading
    kernel argument; a wider stride plans the searched form instead."""
    for T, R in ((256, 256), (2048, 512)):
        rc, p = _plan(lib, T, R, max_blocks=257, bt_rs=(1 << 31) - 1)
        assert rc == 0 and p.request_mode == 3, lib.sconv_last_error()
        rc, p = _plan(lib, T, R, max_blocks=257, bt_rs=1 << 31)
        assert rc == 0 and p.request_mode == 1 and p.bt_row_entries == 0


def test_plan_shapes_of_the_benchmarked_launches(lib):
    """The decode, spec-decode and prefill shapes plan the kernels their
    tuning chose: one-row guessed tiles reading 256 entries ahead for
    decode, four-row guessed tiles for speculative decode, four-row tiles
    with per-row buffers for the prefill; and the per-row form never
    guesses."""
    rc, p = _plan(lib, 256, 256)
    assert rc == 0 and (p.request_mode, p.rows_per_tile, p.bt_row_entries) == (3, 1, 256)
    assert p.lane_elems == 8 and p.stream_hist_loads == 1 and p.waves == 512
    rc, p = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097)
    assert rc == 0 and (p.request_mode, p.rows_per_tile, p.rows_per_request) == (3, 4, 4)
    assert p.bt_row_entries == 0 and p.stream_x_loads == 1
    rc, p = _plan(lib, 20450, 16, H=32, ws=128, D=512, max_blocks=641, folded=False)
    assert rc == 0 and (p.request_mode, p.rows_per_tile, p.tile_major) == (0, 4, 0)
    assert p.waves == 8 * ((20450 + 3) // 4) and p.wg_threads == 256
    rc, p = _plan(lib, 256, 256, folded=False)
    assert rc == 0 and p.request_mode == 0 and p.bt_row_entries == 0
    rc, p = _plan(lib, 256, 256, streams=4)
    assert rc == 0 and p.tile_major == 1 and p.waves == 4 * 256 * 2
    rc, p = _plan(lib, 0, 1)
    assert rc == 0 and p.waves == 0 and p.workgroups == 0 and p.early_inserts == 0
    assert _plan(lib, 10, 2, W=5)[0] == 1 and b"W=5" in lib.sconv_last_error()


def test_plan_early_inserts_only_for_one_generation_decode(lib):
    """Cache inserts go behind the history loads only in one-stream decode
    launches whose waves fit the chip at once (5120 waves of one-row tiles);
    the speculative conv, a layer's four streams, the prefill and larger
    decode batches keep them after the arithmetic."""
    for T, expect in ((256, 1), (1024, 1), (2560, 1), (2561, 0), (4096, 0)):
        rc, p = _plan(lib, T, T, max_blocks=min(4097, T + 1))
        assert rc == 0 and p.rows_per_tile == 1 and p.stream_hist_loads == 1
        assert p.early_inserts == expect, (T, p.waves)
    rc, p = _plan(lib, 256, 256, streams=4)
    assert rc == 0 and p.early_inserts == 0
    rc, p = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097)
    assert rc == 0 and p.rows_per_tile == 4 and p.early_inserts == 0
    rc, p = _plan(lib, 20450, 16, H=32, ws=128, D=512, max_blocks=641, folded=False)
    assert rc == 0 and p.early_inserts == 0
    # whole-line history pieces (no streaming history loads): no early inserts
    rc, p = _plan(lib, 256, 256, H=16, ws=64, D=128)
    assert rc == 0 and p.rows_per_tile == 1 and p.stream_hist_loads == 0 and p.early_inserts == 0


def _gather_struct(conv_dim=4096, max_count=512, d_conv=3, seq_len=2048, src_ss=4096,
                   src_sc=1, dt=1):
    from depthwise_causal_conv1d_amd import _lib
    base = STAND_IN
    src = base + (1 << 46)          # far from every conv buffer of _plan
    out = base + (1 << 47)
    return _lib.WindowGather(src, seq_len, conv_dim, src_ss, src_sc, base, base, max_count,
                             out, conv_dim * d_conv, d_conv)


def test_plan_conv_and_gather_in_one_launch(lib):
    """The speculative step's shape (one generation of four-row tiles,
    16-byte lanes on both sides) runs the gather's workgroups in the conv's
    launch, after the conv's; other shapes launch it after the conv; an
    empty gather is no gather."""
    rc, plain = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097)
    rc, p = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                  gather=_gather_struct())
    assert rc == 0, lib.sconv_last_error()
    assert p.gather_mode == 1 and p.wg_threads == 256
    # one gather workgroup per item (2 x 512: 4096 channels in 256-thread
    # groups of 8-channel lanes)
    assert p.workgroups == plain.workgroups + 1024 and plain.gather_mode == 0
    rc, p = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                  gather=_gather_struct(max_count=21))
    assert rc == 0 and p.workgroups == plain.workgroups + 42
    # decode shape (one-row tiles): its own launch after the conv
    rc, p = _plan(lib, 256, 256, gather=_gather_struct(conv_dim=1024, seq_len=256, src_ss=1024))
    assert rc == 0 and p.gather_mode == 2 and p.workgroups == 512
    # a gather whose source rows are not 16-byte lanes: separate launch
    rc, p = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                  gather=_gather_struct(src_ss=4097))
    assert rc == 0 and p.gather_mode == 2
    # nothing to gather
    rc, p = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                  gather=_gather_struct(max_count=0))
    assert rc == 0 and p.gather_mode == 0
    # no rows: the gather alone
    rc, p = _plan(lib, 0, 512, gather=_gather_struct())
    assert rc == 0 and p.gather_mode == 2 and p.workgroups == 0


def test_combined_entry_rejects_bad_gathers(lib):
    assert _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                 gather=_gather_struct(d_conv=5))[0] == 2
    assert b"d_conv=5" in lib.sconv_last_error()
    assert _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                 gather=_gather_struct(seq_len=0))[0] == 1
    # the gather writing over the conv's input rows
    g = _gather_struct()
    rc, plan = _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097, gather=g)
    assert rc == 0
    g.out = STAND_IN + (1 << 40)     # stream 0's x in _plan
    assert _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                 gather=g)[0] == 1
    assert b"overlaps" in lib.sconv_last_error()
    g.out = STAND_IN                 # the weights, positions and metadata in _plan
    assert _plan(lib, 2048, 512, H=64, ws=64, D=64, N=32, max_blocks=4097,
                 gather=g)[0] == 1
    assert b"overlaps" in lib.sconv_last_error()
