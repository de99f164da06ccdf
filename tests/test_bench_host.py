"""bench.py's host logic on the CPU: the kernel-source digest that decides
whether committed profiles still describe the kernels, the lookup of those
profiles, and the host facts of the CPU baseline."""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_digest_ignores_comments_and_blank_lines():
    a = "int f() {  // one\n\n  return 1; /* two\n lines */\n}\n"
    b = "int f() {\n  return 1;\n}\n"
    assert bench._strip_comments(a) == bench._strip_comments(b)
    assert bench._strip_comments("int g();") != bench._strip_comments(b)


def test_stored_figures_follow_the_digest(tmp_path, monkeypatch):
    k = "fused_insert_conv_kernel"
    digest = bench.kernel_source_digest(k)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "fused_insert_conv_w.md").write_text(
        f"trace_avg_us: 4.500\nkernel_sources: {digest}\n")
    (tmp_path / "counters_w.md").write_text(
        f"hbm_bytes_per_launch: 5205617\nkernel_sources: {digest}\n")
    assert bench.stored_trace(k, "w") == 4.5
    assert bench.stored_traffic("w", k) == 5205617.0
    # another kernel's sources do not match this summary
    assert bench.stored_traffic("w", "update_kernel") is None
    (tmp_path / "fused_insert_conv_w.md").write_text(
        "trace_avg_us: 4.500\nkernel_sources: 0000000000000000\n")
    assert bench.stored_trace(k, "w") is None
    assert bench.stored_trace(k, "missing") is None
    assert bench.stored_traffic("missing", k) is None


def test_kernel_digest_covers_its_source_and_headers():
    assert bench._kernel_sources("fused_insert_conv_kernel") == [
        "fused_insert_conv.hip", "gather_window.h", "sconv_device.h", "sconv_host.h"]
    assert bench._kernel_sources("update_kernel") == [
        "causal_conv1d.hip", "sconv_device.h", "sconv_host.h"]
    assert bench._kernel_sources("gather_ssm_kernel") == [
        "gather_window.h", "gather_window.hip", "sconv_device.h", "sconv_host.h"]
    assert bench.kernel_source_digest("update_kernel") == bench.kernel_source_digest(
        "varlen_fwd_kernel")
    assert bench.kernel_source_digest("update_kernel") != bench.kernel_source_digest(
        "fused_insert_conv_kernel")


def test_committed_profiles_name_their_command_and_digest():
    for name in os.listdir(bench.PROFILES):
        text = open(os.path.join(bench.PROFILES, name)).read()
        assert "rocprofv3" in text and "bench.py" in text, name
        assert "kernel_sources:" in text, name
        if not name.startswith("counters_"):
            assert "trace_avg_us:" in text and "event_us:" in text, name


def test_cpu_threads_honour_the_share(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.cpu_threads() == 1
    monkeypatch.setenv("OMP_NUM_THREADS", "100000")
    assert bench.cpu_threads() == min(n, 256)
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_threads() == min(n, 256)
    assert bench.cpu_model()


def test_repeat_until_spends_the_budget():
    calls = []

    def once(n):
        calls.append(n)
        return 10, 0.25
    tokens, spent, n = bench.repeat_until(1.0, once)
    assert (tokens, spent, n) == (40, 1.0, 4) and calls == [0, 1, 2, 3]
    assert bench.repeat_until(0.0, once)[2] == 1   # at least once


def test_probe_launchers_reject_shapes_they_are_not_built_for():
    """Each streaming probe and the prefill-layout probe checks its shape on
    the host and returns -1 before any HIP call (NULL buffers are never
    touched), so these run without a GPU."""
    import pytest
    if not os.path.exists(bench.PROBE_LIB):
        pytest.skip("bench_probes.so is not built")
    P = bench._probe_lib()
    n = 1 << 16
    # lane depths other than 1, 2 and 4, and empty or non-positive shares
    for u in (0, 3, 8):
        assert P.probe_read(None, n, None, 256, u, 0, None) == -1
        assert P.probe_write(None, n, 256, u, 1, 0, None) == -1
        assert P.probe_copy(None, None, n, 256, u, 1, 0, None) == -1
    assert P.probe_copy(None, None, n, 0, 1, 1, 0, None) == -1
    assert P.probe_write(None, 0, 256, 1, 1, 0, None) == -1
    # more workgroups than a grid holds
    assert P.probe_read(None, 1 << 40, None, 1, 1, 0, None) == -1
    # pieces: multiples of 16 bytes, piece <= row, n a multiple of a piece
    assert P.probe_read_write2(None, None, None, n, 24, 1024, 256, 1, 1, 0, None) == -1
    assert P.probe_read_write2(None, None, None, n, 2048, 1024, 256, 1, 1, 0, None) == -1
    assert P.probe_read_write2(None, None, None, n + 1, 256, 1024, 256, 1, 1, 0, None) == -1
    # the layout probe: T a positive multiple of 16; halo 0 or 3; taps 0 or 4
    for T, halo, wts in ((8, 0, 0), (24, 0, 0), (32, 2, 0), (32, 0, 3)):
        assert P.probe_prefill_layout(None, None, None, None, T, halo, wts, 0, None) == -1
    assert P.probe_chain(None, 0, None, None, None, 1, 17, None) == -1
