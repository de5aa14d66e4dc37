"""Host logic of bench.py that needs no device: the counted-traffic figure it reports is
tied to the library sources it was measured on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_is_reported_only_for_the_profiled_sources(monkeypatch):
    stored = dict(bench.PROFILED_TRAFFIC)
    # a hash of other sources: every kernel reports null
    monkeypatch.setitem(bench.PROFILED_TRAFFIC, "sources_sha256", "0" * 64)
    assert all(bench.profiled_traffic(k) is None for k in stored["bytes"])
    # the stored hash: the stored figure if the sources still match it, else null
    monkeypatch.setitem(bench.PROFILED_TRAFFIC, "sources_sha256", stored["sources_sha256"])
    got = bench.profiled_traffic("down")
    assert got in (None, stored["bytes"]["down"])
    assert bench.profiled_traffic("no_such_kernel") is None


def test_stored_traffic_is_at_least_the_algorithmic_bytes():
    # counted HBM bytes per launch can exceed, never undercut, the operands read once
    assert bench.PROFILED_TRAFFIC["bytes"]["down"] >= 1024 * 4096 * 2        # W_d bf16
    assert bench.PROFILED_TRAFFIC["bytes"]["gate_up"] >= 8192 * 1024 * 2     # W_gu bf16
