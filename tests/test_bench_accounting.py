"""The benchmark's byte accounting, on the CPU.

Algorithmic bytes are what the operator must read or write: token and scale
rows read and written, the top-k weights read and written, permute_token_idx
written, the count matrix read and expert_token_num written. The totals below
are worked out by hand from the workload shapes (the pages' example shape and
four other named workloads), not from the code under test."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_token_re_amd import workloads  # noqa: E402

# name -> (A, token row bytes R, scale row bytes Rs, weight, count bytes, N*E, E)
SHAPES = {
    "pages_shape": (16384, 7168, 4, False, 4, 256, 16),      # int8 rows, [A] f32 scales
    "balanced_bf16": (16384, 14336, 0, True, 8, 256, 16),   # bf16 rows, int64 counts, weights
    "mxfp8_skewed": (32768, 7168, 224, True, 4, 256, 8),     # fp8 rows, e8m0 [A,112,2] scales
    "tiny_segments": (65536, 1024, 128, True, 4, 16384, 64),  # packed fp4 rows, [A,32] f32 scales
    "experts_384": (16384, 7168, 4, True, 4, 384, 24),       # fp8 rows, [A] f32 scales, weights
}
# the same totals written out as numbers
TOTALS = {"pages_shape": 235_078_720, "balanced_bf16": 469_960_832, "mxfp8_skewed": 484_836_384,
          "tiny_segments": 151_847_168, "experts_384": 235_210_336}


def by_hand(name):
    A, R, Rs, weight, cb, M, E = SHAPES[name]
    per_row = 2 * R + 2 * Rs + (8 if weight else 0) + 4
    return A * per_row + M * cb + E * cb, A * per_row


@pytest.mark.parametrize("name", list(SHAPES))
def test_algorithmic_bytes(name):
    w = workloads.make(name)
    call_bytes, gather_bytes = by_hand(name)
    assert call_bytes == TOTALS[name]
    assert w.algorithmic_bytes() == call_bytes
    assert bench.gather_bytes_per_launch(w) == gather_bytes


def test_traffic_needs_matching_source(tmp_path, monkeypatch):
    """The counter summary is used only for its workload, kernel and direction,
    and only while its source hash matches the kernel sources."""
    w = workloads.make("tiny")
    summary = tmp_path / "counters.txt"
    fields = {"workload": "tiny", "direction": "forward", "kernel": "k", "source_hash": bench.kernel_source_hash(),
              "FETCH_SIZE_KiB": "10", "WRITE_SIZE_KiB": "20", "fetch_scale": "2", "write_scale": "1"}
    summary.write_text("".join(f"{k}: {v}\n" for k, v in fields.items()))
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", str(summary))
    assert bench.traffic_from_profile(w, "k") == (10 * 2 + 20 * 1) * 1024
    assert bench.traffic_from_profile(w, "other") is None
    assert bench.traffic_from_profile(w, "k", "inverse") is None
    summary.write_text(summary.read_text().replace(bench.kernel_source_hash(), "0" * 16))
    assert bench.traffic_from_profile(w, "k") is None


def test_rocprof_average_needs_matching_source(tmp_path, monkeypatch):
    """The committed kernel-trace average is reported only for its workload and
    direction, and only while its source hash matches the library's sources."""
    w = workloads.make("tiny")
    summary = tmp_path / "stats.md"
    fields = {"workload": "tiny", "direction": "forward", "source_hash": bench.kernel_source_hash(),
              "average_ns_fused_kernel": "3740.5"}
    summary.write_text("# a summary\n\n" + "".join(f"{k}: {v}\n" for k, v in fields.items()))
    monkeypatch.setattr(bench, "STATS_SUMMARY", str(summary))
    assert bench.rocprof_average_us(w, "fused_kernel") == pytest.approx(3.7405)
    assert bench.rocprof_average_us(w, "stream_gather_kernel") is None
    assert bench.rocprof_average_us(w, "fused_kernel", "inverse") is None
    summary.write_text(summary.read_text().replace(bench.kernel_source_hash(), "0" * 16))
    assert bench.rocprof_average_us(w, "fused_kernel") is None
