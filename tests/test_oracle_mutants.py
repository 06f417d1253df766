"""Plants plausible mistakes in copies of the oracle's C source, builds each
copy on the CPU, and checks that at least one pin (oracle_pins.py) fails for
every one of them. The pins are only worth something if they catch these."""
import os
import subprocess
import sys

import pytest

from oracle import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement). Each text must occur exactly once.
MUTANTS = [
    ("dst_offsets_rank_major",
     "  for (int64_t j = 0; j < E; ++j) {\n    for (int64_t i = 0; i < N; ++i) {\n      dst_off",
     "  for (int64_t i = 0; i < N; ++i) {\n    for (int64_t j = 0; j < E; ++j) {\n      dst_off"),
    ("src_offsets_expert_major",
     "  for (int64_t i = 0; i < N; ++i) {\n    for (int64_t j = 0; j < E; ++j) {\n      src_off",
     "  for (int64_t j = 0; j < E; ++j) {\n    for (int64_t i = 0; i < N; ++i) {\n      src_off"),
    ("src_offsets_inclusive",
     "      src_off[i * E + j] = seen;\n      seen += count_at(counts, counts_is_i64, i * E + j);",
     "      seen += count_at(counts, counts_is_i64, i * E + j);\n      src_off[i * E + j] = seen;"),
    ("dst_offsets_transposed_read",
     "      dst_off[i * E + j] = seen;\n      seen += count_at(counts, counts_is_i64, i * E + j);",
     "      dst_off[i * E + j] = seen;\n      seen += count_at(counts, counts_is_i64, j * N + i);"),
    ("gather_idx_drops_k",
     "out_idx[dst + k] = (int32_t)(src + k);",
     "out_idx[dst + k] = (int32_t)(src);"),
    ("scatter_idx_is_gather",
     "out_idx[src + k] = (int32_t)(dst + k);",
     "out_idx[dst + k] = (int32_t)(src + k);"),
    ("scales_read_at_dst",
     "scales + (src + k) * scale_row_bytes",
     "scales + (dst + k) * scale_row_bytes"),
    ("weight_read_at_dst",
     "weight + (src + k), sizeof(float)",
     "weight + (dst + k), sizeof(float)"),
    ("tokens_one_row_off",
     "tokens + (src + k) * token_row_bytes",
     "tokens + (src + k + (k > 0)) * token_row_bytes"),
    ("cumsum_exclusive",
     "    running += per_expert;\n    int64_t value = (etn_type == 1) ? per_expert : running;",
     "    int64_t value = (etn_type == 1) ? per_expert : running;\n    running += per_expert;"),
    ("etn_row_sums",
     "for (int64_t i = 0; i < N; ++i) per_expert += count_at(counts, counts_is_i64, i * E + j);",
     "for (int64_t i = 0; i < N; ++i) per_expert += count_at(counts, counts_is_i64, j * N + i);"),
    ("inverse_gather_idx_is_scatter",
     "out_idx[rank_row] = (int32_t)expert_row;",
     "out_idx[expert_row] = (int32_t)rank_row;"),
    ("inverse_scatter_idx_drops_k",
     "out_idx[expert_row] = (int32_t)rank_row;",
     "out_idx[expert_row] = (int32_t)src;"),
    ("inverse_moves_forward",
     "memcpy(out_rows + rank_row * row_bytes, rows + expert_row * row_bytes",
     "memcpy(out_rows + expert_row * row_bytes, rows + rank_row * row_bytes"),
    ("inverse_scales_from_rank_row",
     "scales + expert_row * scale_row_bytes",
     "scales + rank_row * scale_row_bytes"),
    ("inverse_weight_from_rank_row",
     "weight + expert_row, sizeof(float)",
     "weight + rank_row, sizeof(float)"),
    ("no_sum_check",
     "  if (total != A) return ORACLE_BAD_COUNTS;\n",
     "  (void)total;\n  (void)A;\n"),
    ("no_negative_check",
     ("    if (c < 0) return ORACLE_BAD_COUNTS;\n",
      "    if (count_at(counts, counts_is_i64, cell) < 0) return ORACLE_BAD_COUNTS;\n"),
     ("", "    (void)cell;\n")),
]


def _sites(old, new):
    return list(zip(old, new)) if isinstance(old, tuple) else [(old, new)]


def test_source_matches_mutant_sites():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        for o, _ in _sites(old, new):
            assert src.count(o) == 1, name


_CHILD = r"""
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
from oracle import oracle
import oracle_pins as pins
orc = oracle.Oracle(sys.argv[1])
failed = []
for name, check in pins.ALL_CHECKS:
    try:
        check(orc)
    except (AssertionError, oracle.OracleError, IndexError, ValueError):
        failed.append(name)
print("failed:", failed)
sys.exit(1 if failed else 0)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    """A planted mistake may also corrupt memory (that is part of the mistake),
    so the pins run against it in a child process: a pin failure or a crash
    there both count as caught; only a clean pass of every pin fails the test."""
    src = open(SRC).read()
    for o, n in _sites(old, new):
        src = src.replace(o, n)
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src)
    lib = oracle.build(str(path), str(tmp_path / f"lib_{name}.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    here = os.path.dirname(os.path.abspath(__file__))
    res = subprocess.run([sys.executable, "-c", _CHILD, lib, root, here], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0, f"mutant {name} passed every pin: {res.stdout}"
