"""Parity at millions of rows, byte for byte against the CPU oracle, through
the C ABI: grids of millions of 64-lane gather workgroups, row maps of
several MiB, offsets kernels with thousands of workgroups (one per 256 rows)
and banded offsets with the largest workgroup split (16 per band, each
walking ~100k source rows), in both directions, with every per-row item
(scales of each layout, weights, both index forms)."""
import pytest

from gpu_helpers import check
from moe_token_re_amd import _lib, workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("direction", [_lib.FORWARD, _lib.INVERSE], ids=["forward", "inverse"])
def test_banded_millions_of_rows(direction):
    # 64 x 32 cells (two bands of 32 ranks), ~3.07M rows of 64 bytes: rows
    # shorter than a 64-vector chunk, so the gather's per-lane row split runs.
    w = workloads.random_case(101, 64, 32, 64, tokens_dtype="int8", count_range=(0, 3000), scales="a",
                              weight=True, idx_type=0)
    assert w.A > 3_000_000
    check(w, direction=direction)


@pytest.mark.parametrize("direction", [_lib.FORWARD, _lib.INVERSE], ids=["forward", "inverse"])
def test_small_matrix_millions_of_rows(direction):
    # 16 x 16 cells, ~2.56M rows of 256 bytes (four rows per 64-vector chunk):
    # ~10k offsets workgroups, MX block scales, scatter index, cumsum counts.
    w = workloads.random_case(102, 16, 16, 128, tokens_dtype="float16", count_range=(0, 20000), scales="e8m0",
                              idx_type=1, etn_type=0)
    assert w.A > 2_000_000
    check(w, direction=direction)


def test_one_cell_many_rows():
    # a single cell (the identity permutation) over 600k rows of exactly one
    # 1 KiB chunk each, [A, 3] fp32 scales, the two phases called apart
    w = workloads.random_case(103, 1, 1, 512, tokens_dtype="bfloat16", count_range=(600_000, 600_001),
                              scales="as", S=3)
    check(w, phases=True)
