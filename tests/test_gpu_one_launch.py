"""Parity of the one-launch stream kernel with the CPU oracle, byte for byte.

moe_rerouting_v2 takes that kernel for count matrices of at most 512 cells,
token rows of 16-byte vectors and at least 32 bytes or of any length from 17
bytes, and scale rows of at most 4 KiB, at any size (short rows only from 2
MiB or 256 KiB of token rows when the fused kernel applies; every case below
first checks, through the plan, that it does): item waves of 64 or 256 output
rows, then one wave per KiB of the input token rows, each wave computing the
offsets it needs from the counts. Rows that are no multiple of 16 bytes, and
rows of 16-byte vectors from 1000 bytes that are no multiple of 64, take its
byte form (the rows as one byte stream, stores grouped by 64-byte pieces of
the output).
Cases cover both directions, int32 and int64 counts, empty cells, one rank or
one expert, count matrices of 8, 35, 64 and 256 cells (four a lane) and of
299, 300, 323, 384 and 512 cells (eight a lane, among them counts in 16-byte
groups that end half-way through a lane and matrices of no whole number of
such groups), both index forms and expert_token_num modes, weights, scale
rows of 4 bytes, 12 bytes, e8m0 and 4000 bytes, rows that are no whole
number of KiB (a wave's KiB then reaches into the next row, often of another
cell), and rows of 32 to 1008 bytes (a wave's KiB spans several rows, often of
several cells, empty ones among them).
Rejected counts (negative, a wrong sum, a count above INT32_MAX, int32
counts whose sum wraps to A modulo 2^32) leave every output untouched."""
import numpy as np
import pytest

from gpu_helpers import SENTINEL, _dev, assert_parity, run_hip, run_oracle
from moe_token_re_amd import _lib, api, workloads

pytestmark = pytest.mark.gpu

MIB = 1 << 20
DIRS = [_lib.FORWARD, _lib.INVERSE]
DIR_IDS = ["forward", "inverse"]


def sized_case(seed, n, e, h, tokens_dtype, target_mib=56, zero_cells=False, **kw):
    """A random case whose token rows total about target_mib MiB."""
    bits = workloads.TOKEN_DTYPES[tokens_dtype][0]
    rows = int(target_mib * MIB) // (h * bits // 8)
    mean = max(1, rows // (n * e))
    lo = 0 if zero_cells else mean // 2
    return workloads.random_case(seed, n, e, h, tokens_dtype=tokens_dtype, count_range=(lo, 2 * mean - lo + 1),
                                 **kw)


def takes_one_launch(w, direction):
    dev = _dev()
    t = workloads.torch_inputs(w, dev)
    call, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"], expert_topk_weight=t["weight"],
                            expert_token_num_type=w.etn_type, idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"],
                            direction=direction)
    return call.plan()["fused"] == 2


CASES = {
    "16x16_int8_a": dict(seed=501, n=16, e=16, h=1024, tokens_dtype="int8", scales="a"),
    "16x16_bf16_i64_w_scatter_cumsum": dict(seed=502, n=16, e=16, h=2048, tokens_dtype="bfloat16",
                                            counts_dtype=np.int64, weight=True, idx_type=1, etn_type=0),
    "32x8_fp8_e8m0_w_scatter": dict(seed=503, n=32, e=8, h=7168, tokens_dtype="float8_e4m3fn", scales="e8m0",
                                    weight=True, idx_type=1),
    "5x7_f16_as3_zeros": dict(seed=504, n=5, e=7, h=512, tokens_dtype="float16", scales="as", S=3, zero_cells=True),
    "1x256_int8": dict(seed=505, n=1, e=256, h=1024, tokens_dtype="int8", weight=True),
    "256x1_fp4_a": dict(seed=506, n=256, e=1, h=4096, tokens_dtype="float4_e2m1fn_x2", scales="a", etn_type=0),
    "8x8_f16_as37_w": dict(seed=507, n=8, e=8, h=512, tokens_dtype="float16", scales="as", S=37, weight=True),
    "16x16_int8_wide_rows_zeros": dict(seed=508, n=16, e=16, h=15360, tokens_dtype="int8", zero_cells=True,
                                       weight=True),
    "4x4_int8_as1000": dict(seed=509, n=4, e=4, h=3072, tokens_dtype="int8", scales="as", S=1000, idx_type=1),
    "16x13_bf16_e8m0_i64": dict(seed=510, n=16, e=13, h=1536, tokens_dtype="bfloat16", scales="e8m0",
                                counts_dtype=np.int64, etn_type=0),
    # rows that are no whole number of KiB
    "16x16_fp8_3584_a": dict(seed=520, n=16, e=16, h=3584, tokens_dtype="float8_e4m3fn", scales="a", target_mib=16),
    "16x16_int8_1040_small_cells": dict(seed=521, n=16, e=16, h=1040, tokens_dtype="int8", zero_cells=True,
                                        weight=True, target_mib=1),
    "8x32_fp8_2880_i64_w_scatter": dict(seed=522, n=8, e=32, h=2880, tokens_dtype="float8_e5m2",
                                        counts_dtype=np.int64, weight=True, idx_type=1, scales="e8m0",
                                        target_mib=24),
    "4x60_bf16_1440_as5_cumsum": dict(seed=523, n=4, e=60, h=720, tokens_dtype="bfloat16", scales="as", S=5,
                                      etn_type=0, target_mib=12),
    "2x4_int8_1040_tiny": dict(seed=524, n=2, e=4, h=1040, tokens_dtype="int8", scales="a", target_mib=0.04),
    "1x1_f16_1040": dict(seed=525, n=1, e=1, h=520, tokens_dtype="float16", weight=True, target_mib=2),
    # 257..512 cells: eight a lane
    "16x32_int8_a": dict(seed=530, n=16, e=32, h=7168, tokens_dtype="int8", scales="a"),
    "24x16_bf16_i64_w_scatter_cumsum": dict(seed=531, n=24, e=16, h=2048, tokens_dtype="bfloat16",
                                            counts_dtype=np.int64, weight=True, idx_type=1, etn_type=0),
    "1x512_int8_w": dict(seed=532, n=1, e=512, h=1024, tokens_dtype="int8", weight=True, zero_cells=True),
    "512x1_fp8_e8m0": dict(seed=533, n=512, e=1, h=4096, tokens_dtype="float8_e4m3fn", scales="e8m0"),
    "17x19_f16_as3_zeros": dict(seed=534, n=17, e=19, h=512, tokens_dtype="float16", scales="as", S=3,
                                zero_cells=True),
    "20x15_int8_1040_w": dict(seed=535, n=20, e=15, h=1040, tokens_dtype="int8", weight=True, target_mib=8),
    "16x32_fp4_as1000_i64_scatter": dict(seed=536, n=16, e=32, h=4096, tokens_dtype="float4_e2m1fn_x2",
                                         scales="as", S=1000, counts_dtype=np.int64, idx_type=1),
    "32x16_fp8_3584_w_cumsum": dict(seed=537, n=32, e=16, h=3584, tokens_dtype="float8_e5m2", weight=True,
                                    etn_type=0, target_mib=20),
    "13x23_bf16_i64_as2_zeros": dict(seed=538, n=13, e=23, h=1024, tokens_dtype="bfloat16", scales="as", S=2,
                                     counts_dtype=np.int64, zero_cells=True, idx_type=1, target_mib=24),
}


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("name", list(CASES))
def test_one_launch_parity(name, direction):
    w = sized_case(**CASES[name])
    assert takes_one_launch(w, direction), name
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("ne", [(16, 16), (16, 32)], ids=["256_cells", "512_cells"])
def test_one_launch_equals_two_phases(ne, direction):
    """The same call through the two phases (offsets kernel, stream gather)."""
    w = sized_case(511, ne[0], ne[1], 1024, "int8", scales="e8m0", weight=True, idx_type=1)
    assert takes_one_launch(w, direction)
    whole, st1 = run_hip(w, _dev(), direction=direction)
    parts, st2 = run_hip(w, _dev(), phases=True, direction=direction)
    assert st1 == st2 == _lib.SUCCESS
    for x, y in zip(whole, parts):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("ne", [(16, 16), (24, 16)], ids=["256_cells", "384_cells"])
@pytest.mark.parametrize("kind", ["negative", "sum_low", "sum_high", "too_large", "wraps"])
def test_one_launch_bad_counts_write_nothing(kind, ne, direction):
    rng = np.random.default_rng(77)
    (n, e), row = ne, 1024
    counts = rng.integers(180, 220, (n, e)).astype(np.int64 if kind == "too_large" else np.int32)
    a = int(counts.sum())
    if kind == "negative":
        counts[1, 1] = -counts[1, 1]
        counts[2, 2] += 2 * abs(int(counts[1, 1]))   # keep the sum at a
    elif kind == "sum_low":
        counts[0, 0] -= 1
    elif kind == "sum_high":
        counts[0, 0] += 1
    elif kind == "too_large":
        counts[3, 2] = (1 << 32) + counts[3, 2]     # above INT32_MAX
    else:
        # two counts at INT32_MAX: the true sum is a + 2^32, its low 32 bits a
        o = int(counts[0, 0]) + int(counts[0, 1])
        counts[0, 0] = counts[0, 1] = (1 << 31) - 1
        counts[0, 2] += o + 2
        assert int(counts.astype(np.int64).sum()) == a + (1 << 32)
    tok = rng.integers(0, 256, (a, row), dtype=np.uint8)
    w = workloads.Workload(f"bad_{kind}", counts, tok, "int8", row,
                           rng.standard_normal(a, dtype=np.float32), "float32",
                           rng.random((a, 1), dtype=np.float32), 1, 0)
    assert takes_one_launch(w, direction)
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.ERROR_BAD_COUNTS, kind
    for o in out:
        assert (o == SENTINEL).all(), kind


def exact_case(seed, n, e, a, row_bytes, scale_words, idx_type):
    """A call of exactly `a` rows over n x e cells (multinomial counts, most
    cells empty when a is small): int8 token rows of row_bytes, [A] or
    [A, scale_words] fp32 scales, weights."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(a, [1.0 / (n * e)] * (n * e)).reshape(n, e).astype(np.int32)
    tok = rng.integers(0, 256, (a, row_bytes), dtype=np.uint8)
    shape = (a,) if scale_words == 1 else (a, scale_words)
    scales = rng.standard_normal(shape, dtype=np.float32)
    weight = rng.random((a, 1), dtype=np.float32)
    return workloads.Workload(f"exact_{seed}_{a}", counts, tok, "int8", row_bytes, scales, "float32", weight, 1,
                              idx_type)


# Item waves move 256 output rows each when scale rows are at most 16 bytes
# (four a lane) and 64 rows otherwise: row counts at and around those
# boundaries, one row, and rows that are no whole number of KiB.
EDGE_ROWS = [(1, 1), (255, 1), (256, 1), (257, 1), (513, 1), (1, 8), (63, 8), (64, 8), (65, 8), (129, 8)]


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("ne", [(16, 16), (16, 24)], ids=["256_cells", "384_cells"])
@pytest.mark.parametrize("a,scale_words", EDGE_ROWS, ids=[f"A{a}_s{s}" for a, s in EDGE_ROWS])
def test_one_launch_item_wave_edges(a, scale_words, ne, direction):
    row_bytes = 1040 if a % 2 else 1024
    w = exact_case(600 + a, ne[0], ne[1], a, row_bytes, scale_words, idx_type=a % 2)
    assert w.A == a
    assert takes_one_launch(w, direction)
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))


def mixed_case(seed, n, e, row_bytes, target_mib, tokens_dtype="int8", small=(0, 4), **kw):
    """Counts mostly small (so that a 1 KiB chunk of short rows spans several
    cells, empty ones among them) with one large cell that brings the token
    rows to about target_mib MiB."""
    rng = np.random.default_rng(seed)
    bits = workloads.TOKEN_DTYPES[tokens_dtype][0]
    h = row_bytes * 8 // bits
    w = workloads.random_case(seed, n, e, h, tokens_dtype=tokens_dtype, count_range=small, **kw)
    counts = w.counts.copy()
    want = int(target_mib * MIB) // row_bytes
    big = int(rng.integers(0, n * e))
    counts.reshape(-1)[big] += max(0, want - int(counts.sum()))
    a = int(counts.sum())
    tok = rng.integers(0, 256, (a, row_bytes), dtype=np.uint8).view(w.tokens.dtype).reshape(a, -1)
    sc = None
    if w.scales is not None:
        sc = rng.integers(0, 256, (a,) + w.scales.shape[1:] + (w.scales.dtype.itemsize,), dtype=np.uint8)
        sc = sc.view(w.scales.dtype).reshape((a,) + w.scales.shape[1:])
    wt = rng.random((a, 1), dtype=np.float32) if w.weight is not None else None
    return workloads.Workload(f"mixed_{seed}", counts, tok, tokens_dtype, h, sc, w.scales_dtype, wt, w.etn_type,
                              w.idx_type)


# Token rows of 16-byte vectors under 1 KiB: a chunk spans several rows, often
# of several cells. Calls of at least 2 MiB of token rows (the fused kernel
# takes smaller ones where it applies), or with more than 256 cells.
SMALL_ROWS = {
    "16x16_32B_mixed": dict(seed=700, n=16, e=16, row_bytes=32, target_mib=3),
    "16x16_48B_mixed_w_scatter": dict(seed=701, n=16, e=16, row_bytes=48, target_mib=3, weight=True, idx_type=1,
                                      scales="a"),
    "5x7_64B_mixed_as3": dict(seed=702, n=5, e=7, row_bytes=64, target_mib=4, scales="as", S=3),
    "16x24_128B_mixed_e8m0": dict(seed=703, n=16, e=24, row_bytes=128, target_mib=1, tokens_dtype="float8_e4m3fn",
                                  scales="e8m0"),
    "64x8_256B_mixed_i64_cumsum": dict(seed=704, n=64, e=8, row_bytes=256, target_mib=2, tokens_dtype="bfloat16",
                                       counts_dtype=np.int64, etn_type=0, weight=True),
    "1x1_512B": dict(seed=705, n=1, e=1, row_bytes=512, target_mib=3, small=(0, 1)),
    "32x8_1008B_mixed_w": dict(seed=706, n=32, e=8, row_bytes=1008, target_mib=6, weight=True, scales="a"),
    "13x23_80B_mixed_i64": dict(seed=707, n=13, e=23, row_bytes=80, target_mib=0.5, counts_dtype=np.int64,
                                small=(0, 3)),
}


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("name", list(SMALL_ROWS))
def test_one_launch_small_rows(name, direction):
    w = mixed_case(**SMALL_ROWS[name])
    assert takes_one_launch(w, direction), name
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
def test_small_rows_below_2mib_stay_fused(direction):
    w = mixed_case(708, 16, 16, 256, 1)
    dev = _dev()
    t = workloads.torch_inputs(w, dev)
    call, _ = api.make_call(t["tokens"], t["counts"], tokens_dtype=t["tokens_dtype"], direction=direction)
    assert call.plan()["fused"] == 1
    out, status = run_hip(w, dev, direction=direction)
    assert status == _lib.SUCCESS
    assert_parity(w, out, run_oracle(w, direction))


# Token rows that are no multiple of 16 bytes (the kernel's byte form): the
# rows as one byte stream, 960 bytes a wave, stores grouped by 64-byte
# segments of the output; a cell's output bytes start and end inside 16-byte
# blocks shared with the cells next to it in the output, whose waves write the
# other bytes. Mostly small cells (a wave's bytes span several cells, empty
# ones among them) with one large cell, as above.
BYTE_ROWS = {
    "16x16_158B_f16_w": dict(seed=720, n=16, e=16, row_bytes=158, target_mib=4, tokens_dtype="float16",
                             weight=True),
    "16x16_17B_i64_scatter": dict(seed=721, n=16, e=16, row_bytes=17, target_mib=3, counts_dtype=np.int64,
                                  idx_type=1),
    "5x7_42B_bf16_as3": dict(seed=722, n=5, e=7, row_bytes=42, target_mib=3, tokens_dtype="bfloat16", scales="as",
                             S=3),
    "16x24_1000B_fp8_e8m0": dict(seed=723, n=16, e=24, row_bytes=1000, target_mib=3, tokens_dtype="float8_e4m3fn",
                                 scales="e8m0"),
    "1x1_1025B_fp4": dict(seed=724, n=1, e=1, row_bytes=1025, target_mib=3, tokens_dtype="float4_e2m1fn_x2",
                          small=(0, 1)),
    "32x16_4097B_w_cumsum": dict(seed=725, n=32, e=16, row_bytes=4097, target_mib=8, weight=True, etn_type=0),
    "64x8_90B_f16_zeros": dict(seed=726, n=64, e=8, row_bytes=90, target_mib=2.5, tokens_dtype="float16",
                               small=(0, 2)),
    "16x16_7169B_a": dict(seed=727, n=16, e=16, row_bytes=7169, target_mib=24, scales="a"),
    "13x23_1009B_i64_as2": dict(seed=728, n=13, e=23, row_bytes=1009, target_mib=6, counts_dtype=np.int64,
                                scales="as", S=2),
    "8x8_30B_f16_cells_to_40": dict(seed=729, n=8, e=8, row_bytes=30, target_mib=2.5, tokens_dtype="float16",
                                    small=(0, 40)),
}


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("name", list(BYTE_ROWS))
def test_one_launch_byte_rows(name, direction):
    w = mixed_case(**BYTE_ROWS[name])
    assert w.tokens.nbytes // w.A % 16 != 0
    assert takes_one_launch(w, direction), name
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))


# Balanced counts (cells of hundreds of rows: most waves lie inside one cell).
BYTE_SIZED = {
    "16x16_f16_H79": dict(seed=730, n=16, e=16, h=79, tokens_dtype="float16", target_mib=40, weight=True),
    "16x32_int8_H1001_zeros": dict(seed=731, n=16, e=32, h=1001, tokens_dtype="int8", zero_cells=True,
                                   target_mib=16, scales="a"),
    "24x16_bf16_H21_i64_scatter": dict(seed=732, n=24, e=16, h=21, tokens_dtype="bfloat16", counts_dtype=np.int64,
                                       idx_type=1, target_mib=4),
    "4x4_fp4_H4098_e8m0_cumsum": dict(seed=733, n=4, e=4, h=4098, tokens_dtype="float4_e2m1fn_x2",
                                      scales="e8m0", etn_type=0, target_mib=12),
    # rows of 16-byte vectors that are no multiple of 64 bytes (the byte form from 1000 bytes)
    "16x16_int8_H7184_w": dict(seed=735, n=16, e=16, h=7184, tokens_dtype="int8", weight=True, target_mib=24),
    "24x16_bf16_H504_i64": dict(seed=736, n=24, e=16, h=504, tokens_dtype="bfloat16", counts_dtype=np.int64,
                                target_mib=8, scales="a"),
}


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("name", list(BYTE_SIZED))
def test_one_launch_byte_rows_balanced(name, direction):
    w = sized_case(**BYTE_SIZED[name])
    assert w.tokens.nbytes // w.A % 64 != 0
    assert takes_one_launch(w, direction), name
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))


# A few rows of 1 KiB or more (no fused kernel there): the last wave's bytes
# end inside a block, and with one row a wave's bytes lie in one or two rows.
BYTE_EDGES = [(1, 1025), (2, 1025), (3, 1031), (7, 2047), (63, 1100), (64, 1111), (65, 1033), (256, 1039),
              (257, 1201)]


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("ne", [(16, 16), (16, 24)], ids=["256_cells", "384_cells"])
@pytest.mark.parametrize("a,row_bytes", BYTE_EDGES, ids=[f"A{a}_R{r}" for a, r in BYTE_EDGES])
def test_one_launch_byte_rows_edges(a, row_bytes, ne, direction):
    w = exact_case(650 + a, ne[0], ne[1], a, row_bytes, 1 + 7 * (a % 2), idx_type=a % 2)
    assert w.A == a
    assert takes_one_launch(w, direction)
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
def test_one_launch_byte_rows_equal_two_phases(direction):
    """The byte form against the two phases' byte stream (the run copy)."""
    w = sized_case(734, 16, 16, 79, "float16", target_mib=20, weight=True, scales="a", idx_type=1)
    assert takes_one_launch(w, direction)
    whole, st1 = run_hip(w, _dev(), direction=direction)
    parts, st2 = run_hip(w, _dev(), phases=True, direction=direction)
    assert st1 == st2 == _lib.SUCCESS
    for x, y in zip(whole, parts):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("kind", ["negative", "sum_high"])
def test_one_launch_byte_rows_bad_counts_write_nothing(kind, direction):
    rng = np.random.default_rng(78)
    counts = rng.integers(180, 220, (16, 16)).astype(np.int32)
    a = int(counts.sum())
    if kind == "negative":
        counts[1, 1] = -counts[1, 1]
        counts[2, 2] += 2 * abs(int(counts[1, 1]))
    else:
        counts[0, 0] += 1
    row = 1001
    tok = rng.integers(0, 256, (a, row), dtype=np.uint8)
    w = workloads.Workload(f"bad_bytes_{kind}", counts, tok, "int8", row,
                           rng.standard_normal(a, dtype=np.float32), "float32",
                           rng.random((a, 1), dtype=np.float32), 1, 0)
    assert takes_one_launch(w, direction)
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.ERROR_BAD_COUNTS, kind
    for o in out:
        assert (o == SENTINEL).all(), kind


# Short rows in small calls with more than 256 cells (no fused kernel there):
# a wave's KiB spans many rows, most cells hold a row or none.
SMALL_BYTE_CALLS = [(1, 17), (5, 30), (100, 42), (1000, 158), (3000, 63)]


@pytest.mark.parametrize("direction", DIRS, ids=DIR_IDS)
@pytest.mark.parametrize("a,row_bytes", SMALL_BYTE_CALLS, ids=[f"A{a}_R{r}" for a, r in SMALL_BYTE_CALLS])
def test_one_launch_byte_rows_small_calls(a, row_bytes, direction):
    w = exact_case(680 + a, 16, 24, a, row_bytes, 1 + 2 * (a % 2), idx_type=a % 2)
    assert w.A == a
    assert takes_one_launch(w, direction)
    out, status = run_hip(w, _dev(), direction=direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, out, run_oracle(w, direction))
