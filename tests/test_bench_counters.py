"""bench.py's use of the committed counter summary (CPU only): a field is reported
only while the kernel's sources are the ones the counters were taken on, and the
summary carries what the bench line reads from it."""
import json

import pytest

import bench


def test_summary_has_the_fields_the_line_reads():
    with open(bench.COUNTERS) as f:
        rec = json.load(f)
    for k in ("samp_stats", "samp_gemm", "samp_combine", "samp_finalize", "attn_partial", "attn_combine"):
        assert rec["kernels"][k]["hbm_bytes"] > 0
        assert len(rec["kernels"][k]["sources_sha256"]) == 64
    g = rec["kernels"]["samp_gemm"]
    assert 0.5 < g["clock_ghz"] < 3.0 and 0.0 < g["mfma_busy"] <= 1.0
    # the scale factors come from the plain copy kernel of known size
    assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0


@pytest.mark.parametrize("field", ["hbm_bytes", "clock_ghz", "mfma_busy"])
def test_fields_are_withheld_when_the_sources_differ(monkeypatch, field):
    with open(bench.COUNTERS) as f:
        stored = json.load(f)["kernels"]["samp_gemm"]
    monkeypatch.setattr(bench, "sources_sha256", lambda kernel: stored["sources_sha256"])
    assert bench.measured_counter("samp_gemm", field) == stored[field]
    monkeypatch.setattr(bench, "sources_sha256", lambda kernel: "0" * 64)
    assert bench.measured_counter("samp_gemm", field) is None
    assert bench.measured_traffic("samp_gemm") is None


def test_unknown_kernel_reports_nothing():
    assert bench.measured_counter("no_such_kernel", "hbm_bytes") is None
