"""Pins of the CPU oracle: checks against facts the pages and the mathematics fix,
independent of the oracle's own code.

Each check takes an `Oracle` instance (oracle/oracle.py) and raises
AssertionError on a mismatch, so the same checks run against the real oracle
(test_oracle_pins.py) and against deliberately broken builds of it
(test_oracle_mutants.py, which shows every planted mistake is caught).

What pins what (page: "CANN ops-transformer MoeReRoutingV2", nlpx.cn):
  * golden fixtures     -- hand-worked offsets, both index forms and both
                           expert_token_num modes (section 计算公式, 参数说明);
  * stable-sort brute force -- every count matrix with N, E <= 3 and entries
                           in {0,1,2}: the rank-major input is the rows
                           labelled (rank, expert) in row-major cell order;
                           expert-major order is a stable sort of those labels
                           by (expert, rank), computed by numpy.lexsort;
  * single rank / single expert -> identity; uniform counts -> a block
    transpose done by numpy reshape/transpose;
  * the article's example counts (all ones, 16x16; section 注意) -> a 16x16
    transpose; the V1 page's example (all ones but the last cell) -> a 255-row
    transpose followed by fixed points;
  * invariants: the index is a permutation, gather and scatter forms are
    inverse, scales and weights move with the token rows byte for byte,
    expert_token_num equals the per-expert histogram of the moved rows.
The inverse re-route (expert-major rows back to rank-major order; the page
gives only the forward moves, the inverse reads them backwards) is pinned by:
  * the golden fixtures read backwards: input row d goes to output row
    gather_idx[d], so the inverse's gather index is the fixture's scatter
    index and its scatter index is the fixture's gather index;
  * the stable-sort brute force: the inverse permutation of the sort's
    (numpy argsort of the lexsort order) for every small count matrix;
  * round trips: forward then inverse, and inverse then forward, give back
    the input bytes (tokens, scales, weights) for random count matrices.
"""
from __future__ import annotations

import itertools
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    fields = {}
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            fields[key] = np.array([int(v) for v in vals], np.int64)
    n, e = int(fields["N"][0]), int(fields["E"][0])
    fields["counts"] = fields["counts"].reshape(n, e)
    fields["src_off"] = fields["src_off"].reshape(n, e)
    fields["dst_off"] = fields["dst_off"].reshape(n, e)
    return fields


GOLDEN_FILES = sorted(f for f in os.listdir(GOLDEN_DIR) if f.endswith(".txt"))


def row_coded_tokens(a, row_bytes=8, seed=0):
    """Token rows whose bytes identify the row: the row number in the first four
    bytes (little endian), random bytes after that."""
    rng = np.random.default_rng(seed)
    t = rng.integers(0, 256, (a, max(row_bytes, 4)), dtype=np.uint8)
    t[:, :4] = np.arange(a, dtype=np.uint32).view(np.uint8).reshape(a, 4)
    return t


def labels(counts):
    """(rank, expert) label of every row of the rank-major input: cell (i, j)
    contributes counts[i, j] rows, cells in row-major order."""
    n, e = counts.shape
    flat = counts.reshape(-1).astype(np.int64)
    cell = np.repeat(np.arange(n * e), flat)
    return cell // e, cell % e


def stable_sort_gather(counts):
    """Expert-major order as a stable sort of the row labels by (expert, rank)."""
    rank, expert = labels(counts)
    return np.lexsort((rank, expert))


def check_golden(orc, name):
    g = load_golden(name)
    counts = g["counts"].astype(np.int32)
    src, dst = orc.offsets(counts)
    assert np.array_equal(src, g["src_off"]), (name, src, g["src_off"])
    assert np.array_equal(dst, g["dst_off"]), (name, dst, g["dst_off"])
    a = int(g["A"][0])
    tok = row_coded_tokens(a)
    for idx_type, key in ((0, "gather_idx"), (1, "scatter_idx")):
        for etn_type, ekey in ((1, "etn_count"), (0, "etn_cumsum")):
            out, _, idx, etn, _ = orc.reroute(tok, counts, etn_type=etn_type, idx_type=idx_type)
            assert np.array_equal(idx, g[key]), (name, key, idx)
            assert np.array_equal(etn, g[ekey]), (name, ekey, etn)
            assert np.array_equal(out, tok[g["gather_idx"]]), (name, "tokens")


def check_case_against_sort(orc, counts, row_bytes=5, seed=0, with_extras=True):
    """Every output of one case against the stable-sort construction."""
    a = int(counts.sum())
    tok = row_coded_tokens(a, row_bytes, seed)
    rng = np.random.default_rng(seed + 1)
    scales = rng.integers(0, 256, (a, 12), dtype=np.uint8) if with_extras else None
    weight = rng.integers(0, 256, (a, 4), dtype=np.uint8).view(np.float32).reshape(a, 1) if with_extras else None
    g = stable_sort_gather(counts)
    rank, expert = labels(counts)
    per_expert = np.bincount(expert[g], minlength=counts.shape[1]) if a else np.zeros(counts.shape[1], np.int64)
    for idx_type in (0, 1):
        for etn_type in (0, 1):
            out, o_sc, idx, etn, o_w = orc.reroute(tok, counts, scales, weight, etn_type, idx_type)
            assert np.array_equal(out, tok[g]), ("tokens", counts)
            if idx_type == 0:
                assert np.array_equal(idx, g), ("gather", counts, idx, g)
            else:
                inv = np.empty_like(g)
                inv[g] = np.arange(a)
                assert np.array_equal(idx, inv), ("scatter", counts, idx, inv)
            if with_extras:
                assert np.array_equal(o_sc, scales[g]), ("scales", counts)
                assert np.array_equal(o_w.view(np.uint32), weight.view(np.uint32)[g]), ("weight", counts)
            want = per_expert if etn_type == 1 else np.cumsum(per_expert)
            assert np.array_equal(etn.astype(np.int64), want), ("etn", etn_type, counts, etn, want)


def check_bruteforce(orc, max_n=3, max_e=3, values=(0, 1, 2)):
    """Every count matrix with 1 <= N <= max_n, 1 <= E <= max_e, entries in `values`."""
    cases = 0
    for n in range(1, max_n + 1):
        for e in range(1, max_e + 1):
            for flat in itertools.product(values, repeat=n * e):
                counts = np.array(flat, np.int32).reshape(n, e)
                check_case_against_sort(orc, counts, row_bytes=4, with_extras=(cases % 7 == 0))
                cases += 1
    return cases


def check_identity(orc, seed=0):
    """One rank or one expert: rank-major and expert-major orders coincide."""
    rng = np.random.default_rng(seed)
    for shape in ((1, 7), (9, 1), (1, 1)):
        counts = rng.integers(0, 9, shape).astype(np.int32)
        a = int(counts.sum())
        tok = row_coded_tokens(a, 6)
        out, _, idx, _, _ = orc.reroute(tok, counts)
        assert np.array_equal(idx, np.arange(a)), (shape, idx)
        assert np.array_equal(out, tok)
        _, _, sidx, _, _ = orc.reroute(tok, counts, idx_type=1)
        assert np.array_equal(sidx, np.arange(a))


def check_block_transpose(orc):
    """Equal counts c in every cell: the output is the [N, E, c, R] input with
    the rank and expert axes swapped (numpy transpose)."""
    for n, e, c, r in ((3, 5, 2, 6), (4, 4, 3, 8), (2, 7, 1, 5)):
        counts = np.full((n, e), c, np.int64)
        a = n * e * c
        tok = row_coded_tokens(a, r)
        want = tok.reshape(n, e, c, -1).transpose(1, 0, 2, 3).reshape(a, -1)
        out, _, _, etn, _ = orc.reroute(tok, counts)
        assert np.array_equal(out, want), (n, e, c)
        assert np.array_equal(etn, np.full(e, n * c)), etn


def check_pages_examples(orc):
    """The article's example count matrix is torch.ones(16, 16) (A = 256, as
    its note says): expert-major order is then the 16x16 transpose. The V1
    page's generator (every draw overridden by 1, last cell = remainder) gives
    ones and counts[15,15] = 16384 - 255: the first 255 output rows are that
    transpose without its last entry, and every row from 255 on is fixed."""
    counts = np.ones((16, 16), np.int32)
    tok = row_coded_tokens(256, 4)
    _, _, idx, etn, _ = orc.reroute(tok, counts)
    d = np.arange(256)
    assert np.array_equal(idx, (d % 16) * 16 + d // 16), idx
    assert np.array_equal(etn, np.full(16, 16))

    counts = np.ones((16, 16), np.int32)
    counts[15, 15] = 16384 - 255
    tok = row_coded_tokens(16384, 4)
    _, _, idx, etn, _ = orc.reroute(tok, counts)
    d = np.arange(16384)
    want = np.where(d < 255, (d % 16) * 16 + d // 16, d)
    assert np.array_equal(idx, want)
    assert int((idx == d).sum()) == 16144
    assert np.array_equal(etn, np.r_[np.full(15, 16), 16 + 16128])


def check_random_invariants(orc, seeds=range(6)):
    """Larger random cases (with empty cells): the sort construction again, plus
    the index being a permutation and the two forms being inverses."""
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        n, e = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        dt = np.int32 if seed % 2 else np.int64
        counts = rng.integers(0, 9, (n, e)).astype(dt)
        a = int(counts.sum())
        check_case_against_sort(orc, counts, row_bytes=3 + seed, seed=seed)
        tok = row_coded_tokens(a, 4)
        _, _, g, _, _ = orc.reroute(tok, counts, idx_type=0)
        _, _, s, _, _ = orc.reroute(tok, counts, idx_type=1)
        assert np.array_equal(np.sort(g), np.arange(a))
        assert np.array_equal(g[s], np.arange(a)) and np.array_equal(s[g], np.arange(a))


def check_errors(orc):
    """Invalid counts are rejected and nothing is written."""
    from oracle.oracle import BAD_ARGS, BAD_COUNTS, OracleError

    def expect(code, tok, counts, **kw):
        outs = tuple(None if x is None else x for x in
                     (np.full_like(tok, 0xAB), None, np.full(tok.shape[0], -7, np.int32),
                      np.full(counts.shape[1], -7, counts.dtype), None))
        try:
            orc.reroute(tok, counts, out=outs, **kw)
        except OracleError as err:
            assert err.code == code, (err.code, code)
        else:
            raise AssertionError("accepted bad input")
        assert (outs[0] == 0xAB).all() and (outs[2] == -7).all() and (outs[3] == -7).all()

    tok = row_coded_tokens(6, 4)
    expect(BAD_COUNTS, tok, np.array([[2, -1], [3, 2]], np.int32))   # negative
    expect(BAD_COUNTS, tok, np.array([[2, 1], [3, 1]], np.int32))    # sums to 7, A = 6
    expect(BAD_COUNTS, tok, np.array([[1, 1], [1, 1]], np.int64))    # sums to 4
    expect(BAD_ARGS, tok, np.array([[2, 1], [2, 1]], np.int32), etn_type=2)
    expect(BAD_ARGS, tok, np.array([[2, 1], [2, 1]], np.int32), idx_type=-1)


def check_empty(orc):
    """A = 0: all-zero counts, and degenerate N = 0 / E = 0 matrices."""
    tok = np.zeros((0, 4), np.uint8)
    out, _, idx, etn, _ = orc.reroute(tok, np.zeros((3, 2), np.int32), etn_type=0)
    assert idx.shape == (0,) and np.array_equal(etn, [0, 0])
    _, _, idx, etn, _ = orc.reroute(tok, np.zeros((0, 5), np.int32))
    assert np.array_equal(etn, np.zeros(5))
    _, _, idx, etn, _ = orc.reroute(tok, np.zeros((4, 0), np.int64))
    assert etn.shape == (0,)


def check_inverse_golden(orc, name):
    g = load_golden(name)
    counts = g["counts"].astype(np.int32)
    a = int(g["A"][0])
    rows = row_coded_tokens(a, 6, seed=3)
    for idx_type, key in ((0, "scatter_idx"), (1, "gather_idx")):
        for etn_type, ekey in ((1, "etn_count"), (0, "etn_cumsum")):
            out, _, idx, etn, _ = orc.reroute_inverse(rows, counts, etn_type=etn_type, idx_type=idx_type)
            assert np.array_equal(idx, g[key]), (name, "inverse", key, idx)
            assert np.array_equal(etn, g[ekey]), (name, "inverse", ekey, etn)
            assert np.array_equal(out, rows[g["scatter_idx"]]), (name, "inverse rows")


def check_inverse_case_against_sort(orc, counts, row_bytes=5, seed=0, with_extras=True):
    """Every output of one inverse case against the inverse of the stable-sort order."""
    a = int(counts.sum())
    rows = row_coded_tokens(a, row_bytes, seed)
    rng = np.random.default_rng(seed + 2)
    scales = rng.integers(0, 256, (a, 8), dtype=np.uint8) if with_extras else None
    weight = rng.integers(0, 256, (a, 4), dtype=np.uint8).view(np.float32).reshape(a, 1) if with_extras else None
    g = stable_sort_gather(counts)  # forward: expert-major row d <- rank-major row g[d]
    back = np.argsort(g, kind="stable")  # inverse: rank-major row s <- expert-major row back[s]
    _, expert = labels(counts)
    per_expert = np.bincount(expert, minlength=counts.shape[1]) if a else np.zeros(counts.shape[1], np.int64)
    for idx_type in (0, 1):
        for etn_type in (0, 1):
            out, o_sc, idx, etn, o_w = orc.reroute_inverse(rows, counts, scales, weight, etn_type, idx_type)
            assert np.array_equal(out, rows[back]), ("inverse rows", counts)
            assert np.array_equal(idx, back if idx_type == 0 else g), ("inverse idx", idx_type, counts, idx)
            if with_extras:
                assert np.array_equal(o_sc, scales[back]), ("inverse scales", counts)
                assert np.array_equal(o_w.view(np.uint32), weight.view(np.uint32)[back]), ("inverse weight", counts)
            want = per_expert if etn_type == 1 else np.cumsum(per_expert)
            assert np.array_equal(etn.astype(np.int64), want), ("inverse etn", etn_type, counts)


def check_inverse_bruteforce(orc, max_n=3, max_e=3, values=(0, 1, 2)):
    cases = 0
    for n in range(1, max_n + 1):
        for e in range(1, max_e + 1):
            for flat in itertools.product(values, repeat=n * e):
                counts = np.array(flat, np.int64 if cases % 2 else np.int32).reshape(n, e)
                check_inverse_case_against_sort(orc, counts, row_bytes=4, with_extras=(cases % 5 == 0))
                cases += 1
    return cases


def check_roundtrip(orc, seeds=range(5)):
    """Forward then inverse, and inverse then forward, are the identity."""
    for seed in seeds:
        rng = np.random.default_rng(300 + seed)
        n, e = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        counts = rng.integers(0, 7, (n, e)).astype(np.int32 if seed % 2 else np.int64)
        a = int(counts.sum())
        tok = row_coded_tokens(a, 9, seed)
        scales = rng.integers(0, 256, (a, 3), dtype=np.uint8)
        weight = rng.integers(0, 256, (a, 4), dtype=np.uint8).view(np.float32).reshape(a, 1)
        f_tok, f_sc, f_gidx, _, f_w = orc.reroute(tok, counts, scales, weight, 1, 0)
        b_tok, b_sc, b_sidx, _, b_w = orc.reroute_inverse(f_tok, counts, f_sc, f_w, 1, 1)
        assert np.array_equal(b_tok, tok) and np.array_equal(b_sc, scales), ("round trip", seed)
        assert np.array_equal(b_w.view(np.uint32), weight.view(np.uint32)), ("round trip weight", seed)
        assert np.array_equal(b_sidx, f_gidx), ("inverse scatter idx = forward gather idx", seed)
        y = row_coded_tokens(a, 7, seed + 1)
        assert np.array_equal(orc.reroute(orc.reroute_inverse(y, counts)[0], counts)[0], y), ("inverse then forward",)


def check_inverse_errors(orc):
    from oracle.oracle import BAD_ARGS, BAD_COUNTS, OracleError
    rows = row_coded_tokens(6, 4)
    for counts, code, kw in ((np.array([[2, -1], [3, 2]], np.int32), BAD_COUNTS, {}),
                             (np.array([[2, 1], [3, 1]], np.int64), BAD_COUNTS, {}),
                             (np.array([[2, 1], [2, 1]], np.int32), BAD_ARGS, {"idx_type": 2})):
        outs = (np.full_like(rows, 0xAB), None, np.full(6, -7, np.int32), np.full(2, -7, counts.dtype), None)
        try:
            orc.reroute_inverse(rows, counts, out=outs, **kw)
        except OracleError as err:
            assert err.code == code
        else:
            raise AssertionError("inverse accepted bad input")
        assert (outs[0] == 0xAB).all() and (outs[2] == -7).all() and (outs[3] == -7).all()


ALL_CHECKS = [
    ("golden", lambda o: [check_golden(o, f) for f in GOLDEN_FILES]),
    ("bruteforce", lambda o: check_bruteforce(o, 2, 2, (0, 1, 2))),
    ("identity", check_identity),
    ("block_transpose", check_block_transpose),
    ("pages_examples", check_pages_examples),
    ("random_invariants", check_random_invariants),
    ("errors", check_errors),
    ("empty", check_empty),
    ("inverse_golden", lambda o: [check_inverse_golden(o, f) for f in GOLDEN_FILES]),
    ("inverse_bruteforce", lambda o: check_inverse_bruteforce(o, 2, 2, (0, 1, 2))),
    ("roundtrip", check_roundtrip),
    ("inverse_errors", check_inverse_errors),
]
