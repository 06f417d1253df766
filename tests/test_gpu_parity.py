"""Parity of the HIP path (through the C ABI) with the CPU oracle, byte for byte.

Every output the operator defines is compared raw-byte-exact (tolerance 0: the
operator only moves bytes and computes integer offsets), on seeded inputs:
  * the five named workloads at their full sizes, in the launch configuration
    the benchmark times;
  * a seeded fuzz over the contract: token widths 16/8/4 bits, int32/int64
    counts, scale layouts [A] / [A,S] / e8m0, weights on/off, both index forms,
    both expert_token_num modes, empty segments, odd row sizes and unaligned
    rows, the (N, E) pairs and (A, H) shapes the article's tests name;
  * edge cases: A = 0, N = 0, one rank, one expert, count tables too large
    for LDS, long runs of empty cells;
  * device-detected count errors: outputs are left untouched.
permute_per_token_scales is not compared when no scales are given: the
operator defines no value for it then."""
import numpy as np
import pytest
import torch

from gpu_helpers import SENTINEL, _bytes, _dev, assert_parity, check, run_hip, run_oracle
from moe_token_re_amd import _lib, api, workloads

pytestmark = pytest.mark.gpu


# --- the five named workloads, full size ---------------------------------

@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_named_workload_full_size(name):
    check(workloads.make(name))


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_two_phases_equal_oracle(name):
    """The offsets kernel then the gather kernel, called separately (the
    two-kernel path, also for count matrices small enough for the fused one)."""
    check(workloads.make(name), phases=True)


@pytest.mark.parametrize("seed,n,e", [(1, 2, 4), (2, 16, 16), (3, 1, 40), (4, 33, 3), (5, 9, 1)])
def test_fused_equals_two_phase(seed, n, e):
    """Small count matrices: the single-kernel whole call and the two-kernel
    phases give the same bytes (and both match the oracle)."""
    dev = _dev()
    w = workloads.random_case(seed, n, e, 96, tokens_dtype="bfloat16", count_range=(0, 12), scales="as", S=5,
                              weight=True, idx_type=seed % 2, etn_type=seed % 2)
    t = workloads.torch_inputs(w, dev)
    call, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"], expert_topk_weight=t["weight"],
                            expert_token_num_type=w.etn_type, idx_type=w.idx_type)
    assert call.plan()["fused"] == 1
    whole, st1 = run_hip(w, dev)
    parts, st2 = run_hip(w, dev, phases=True)
    assert st1 == st2 == _lib.SUCCESS
    for x, y in zip(whole, parts):
        assert np.array_equal(x, y)
    assert_parity(w, whole, run_oracle(w))


# --- seeded fuzz over the contract ----------------------------------------

TOKEN_KINDS = ["float16", "bfloat16", "int8", "float8_e5m2", "float8_e4m3fn", "hifloat8",
               "float4_e2m1fn_x2", "float4_e1m2fn_x2"]


def fuzz_cases():
    rng = np.random.default_rng(2024)
    cases = []
    ne_pairs = [(4, 2), (23, 2), (14, 1), (2, 4), (16, 16), (7, 13), (1, 9), (33, 5)]
    for k in range(48):
        n, e = ne_pairs[k % len(ne_pairs)]
        tok = TOKEN_KINDS[k % len(TOKEN_KINDS)]
        h = int(rng.choice([2, 8, 64, 79, 128, 130, 1000, 2048, 7168, 16382]))
        if tok.startswith("float4") and h % 2:
            h += 1
        scales = [None, "a", "as", "e8m0"][k % 4]
        cases.append(dict(seed=1000 + k, N=n, E=e, H=h, tokens_dtype=tok,
                          counts_dtype=np.int64 if k % 3 == 0 else np.int32,
                          count_range=(0, 9) if k % 2 else (1, 40), scales=scales,
                          S=int(rng.integers(1, 40)), weight=bool(k % 5 != 0),
                          etn_type=int(k % 7 == 0) ^ 1, idx_type=int(k % 2 == 1)))
    return cases


@pytest.mark.parametrize("case", fuzz_cases(), ids=lambda c: f"s{c['seed']}")
def test_fuzz(case):
    w = workloads.random_case(**case)
    check(w)               # small calls: the single fused kernel
    check(w, phases=True)  # the two phases: the stream gather where the row map is written


# The largest H the contract allows ("约束说明": 0 < H < 16384): 16383 for
# 8- and 16-bit tokens (rows of 16383 and 32766 bytes, no multiple of 16: the
# byte stream in the two-kernel path), 16382 for packed fp4 (H must be even).
@pytest.mark.parametrize("tok", ["int8", "float16", "bfloat16", "float8_e4m3fn", "float4_e2m1fn_x2"])
def test_largest_h(tok):
    h = 16382 if tok.startswith("float4") else 16383
    w = workloads.random_case(7000 + len(tok), 3, 5, h, tokens_dtype=tok, count_range=(0, 9), scales="e8m0",
                              weight=True, idx_type=len(tok) % 2)
    check(w)
    check(w, phases=True)


# Shapes named by the article's tests ("测试与验证"): (52, 21), (35, 15267),
# (28, 6057), read both ways as (A, H); (N, E) in {(4,2), (23,2), (14,1)}.
@pytest.mark.parametrize("a,h", [(52, 21), (21, 52), (35, 15267), (15267, 35), (28, 6057), (6057, 28)])
@pytest.mark.parametrize("ne", [(4, 2), (23, 2), (14, 1)])
def test_article_test_shapes(a, h, ne):
    n, e = ne
    rng = np.random.default_rng(a * 7 + h)
    # counts >= 0 summing to a: a multinomial over the n*e cells
    counts = rng.multinomial(a, [1.0 / (n * e)] * (n * e)).reshape(n, e).astype(np.int32)
    raw = rng.integers(0, 256, (a, 2 * h), dtype=np.uint8)
    w = workloads.Workload(f"article_{a}x{h}_{n}x{e}", counts, raw.view(np.float16), "float16", h,
                           rng.standard_normal(a, dtype=np.float32), "float32",
                           rng.random((a, 1), dtype=np.float32), 1, (a + h) % 2)
    check(w)


def test_geir_sample_shape():
    """Graph-mode sample: A=11, H=79, N=11, E=1, S=1 (scales [A, 1] f32)."""
    rng = np.random.default_rng(11)
    counts = np.ones((11, 1), np.int32)
    w = workloads.Workload("geir", counts, rng.standard_normal((11, 79)).astype(np.float16), "float16", 79,
                           rng.standard_normal((11, 1), dtype=np.float32), "float32",
                           rng.random((11, 1), dtype=np.float32), 1, 0)
    check(w)


# --- edge cases -----------------------------------------------------------

def test_empty_all_zero_counts():
    w = workloads.random_case(7, 5, 3, 64, count_range=(0, 1))
    assert w.A == 0
    check(w)


def test_zero_ranks():
    w = workloads.Workload("n0", np.zeros((0, 6), np.int64), np.zeros((0, 32), np.float16), "float16", 32,
                           etn_type=0)
    check(w)


@pytest.mark.parametrize("shape", [(1, 300), (300, 1), (1, 1)])
def test_single_rank_or_expert(shape):
    check(workloads.random_case(31, shape[0], shape[1], 256, tokens_dtype="bfloat16", count_range=(0, 7),
                                scales="as", S=3, weight=True, idx_type=1))


def test_large_table_unstaged():
    """N*E = 131072 cells (the largest matrix the banded offsets kernel
    takes), mostly empty, so the row search runs across long stretches of
    empty cells."""
    rng = np.random.default_rng(77)
    counts = np.zeros((512, 256), np.int32)
    cells = rng.choice(512 * 256, 900, replace=False)
    counts.reshape(-1)[cells] = rng.integers(1, 30, 900)
    a = int(counts.sum())
    tok = rng.integers(0, 256, (a, 96), dtype=np.uint8)
    w = workloads.Workload("large_table", counts, tok, "int8", 96, None, None,
                           rng.random((a, 1), dtype=np.float32), 0, 0)
    check(w)


def _offsets_workgroups(w, dev):
    t = workloads.torch_inputs(w, dev)
    call, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"], expert_topk_weight=t["weight"],
                            expert_token_num_type=w.etn_type, idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"])
    return call.plan()["offsets_workgroups"]


# Count matrices of every size class of the single-workgroup offsets kernel
# (taken when the banded kernel does not apply: at most 1024 cells, more than
# 1024 experts, or more than 2^17 cells): one cell per thread, chunks of 3, 5,
# 9 and 17 cells per thread (each class's lower and upper edge), and beyond
# 17408 cells the path through global memory.
@pytest.mark.parametrize("n,e", [(32, 32), (1, 1024), (2, 1025), (1, 3000), (4, 1280), (3, 1700), (5, 1100),
                                 (8, 1152), (9, 1100), (16, 1088), (17, 1025), (130, 1040), (520, 256),
                                 (17, 16), (16, 32), (32, 16), (1, 512), (513, 1), (19, 27)])
def test_offsets_single_workgroup(n, e):
    w = workloads.random_case(n * 7 + e, n, e, 40, tokens_dtype="int8", count_range=(0, 4), weight=True,
                              idx_type=(n + e) % 2, etn_type=(n * e) % 2)
    # one workgroup; with the row map (one cell per thread), one per 256 rows up to 256 cells, one
    # per 512 rows up to 512 cells, else one per 1024 rows
    rows = 256 if n * e <= 256 else 512 if n * e <= 512 else 1024
    want = 1 if n * e > 1024 else max(1, -(-w.A // rows))
    assert _offsets_workgroups(w, _dev()) == want
    check(w)
    check(w, phases=True)


# The banded offsets kernel (1024 < N*E <= 2^17 cells, E <= 1024): one
# workgroup per band of min(N, 1024 // E) ranks, ragged last bands, one rank
# per band (E > 512), one expert, and the largest matrix it takes.
@pytest.mark.parametrize("n,e", [(32, 33), (33, 32), (64, 48), (64, 49), (100, 51), (128, 41), (96, 96),
                                 (97, 96), (136, 128), (137, 128), (256, 64), (5000, 1), (1100, 1), (2, 1024),
                                 (7, 513), (5, 300), (64, 17), (130, 1008), (512, 256)])
def test_offsets_banded(n, e):
    w = workloads.random_case(n * 5 + e, n, e, 40, tokens_dtype="int8", count_range=(0, 4), weight=True,
                              idx_type=(n * e) % 2, etn_type=(n + e) % 2)
    band_rows = min(n, 1024 // e)
    bands = -(-n // band_rows)
    split = min(16, max(1, 2 * w.A // (bands * 1024)))  # workgroups sharing a band's row map writes
    assert _offsets_workgroups(w, _dev()) == bands * split
    check(w)
    check(w, phases=True)


def test_offsets_banded_int64_cumsum():
    w = workloads.random_case(4242, 300, 20, 24, tokens_dtype="float16", counts_dtype="int64", count_range=(0, 6),
                              scales="a", weight=True, idx_type=1, etn_type=0)
    assert _offsets_workgroups(w, _dev()) > 1
    check(w)
    check(w, phases=True)


# The banded kernel writes the row map cell by cell: a thread for cells of up
# to 16 rows, a wave for cells of up to 1024 rows, every workgroup of the band
# for larger ones. Mixed cell sizes put cells in all three classes, in several
# bands and both directions.
@pytest.mark.parametrize("direction", [_lib.FORWARD, _lib.INVERSE], ids=["forward", "inverse"])
def test_offsets_banded_cell_sizes(direction):
    rng = np.random.default_rng(77)
    counts = rng.integers(0, 4, (64, 48)).astype(np.int32)
    mid = rng.choice(counts.size, 60, replace=False)
    counts.flat[mid] = rng.integers(17, 1025, 60)
    counts[5, 7] = 5000        # larger than a workgroup
    counts[40, 47] = 1025      # just above a wave's class
    counts[33, 0] = 16         # the largest per-thread cell
    counts[33, 1] = 17         # the smallest per-wave cell
    a = int(counts.sum())
    w = workloads.Workload("banded_cell_sizes", counts, rng.integers(-128, 128, (a, 48), dtype=np.int8), "int8", 48,
                           rng.standard_normal(a, dtype=np.float32), "float32", rng.random((a, 1), dtype=np.float32),
                           1, int(direction))
    assert _offsets_workgroups(w, _dev()) > 1
    check(w, direction=direction)
    check(w, phases=True, direction=direction)


# Rejected counts are seen by every workgroup of the banded kernel (each
# reads the whole matrix); the bad cell sits in a band other than the first.
@pytest.mark.parametrize("n,e,kind", [(64, 49, "negative"), (97, 96, "negative"), (256, 64, "too_large"),
                                      (256, 64, "sum_high"), (130, 1008, "sum_low"), (2, 1500, "negative"),
                                      (9, 1100, "negative"), (520, 256, "sum_high")])
def test_bad_counts_large(n, e, kind):
    dev = _dev()
    rng = np.random.default_rng(n + e)
    counts = rng.integers(0, 4, (n, e)).astype(np.int64)
    counts[n - 1, e - 1] += 2
    a = int(counts.sum())
    if kind == "negative":
        counts[n // 2, e // 3] = -1  # the sum no longer matches either
    elif kind == "too_large":
        counts[n - 1, e // 2] += 1 << 32  # the sum's low 32 bits still equal a
    elif kind == "sum_high":
        counts[n - 1, 0] += 1
    else:
        counts[n - 1, e - 1] -= 1
    w = workloads.Workload(f"bad_{kind}_{n}x{e}", counts, rng.integers(0, 256, (a, 8), dtype=np.uint8), "int8", 8)
    for phases in (False, True):
        out, status = run_hip(w, dev, phases=phases)
        assert status == _lib.ERROR_BAD_COUNTS
        for o in out:
            assert (o == SENTINEL).all()


@pytest.mark.parametrize("h,tok,scales,S,inline", [
    (64, "float16", "as", 5, 0),       # 256 rows x 5 pieces > threads: separate scale pass
    (64, "float16", "a", 1, 4),        # [A] f32: one 4-byte piece per row
    (7168, "int8", "e8m0", 1, 16),     # 224-byte e8m0 rows: 16-byte pieces
    (2048, "bfloat16", "as", 32, 16),  # 128-byte rows: 16-byte pieces
    (2048, "bfloat16", "as", 3, 4),    # 12-byte rows: 4-byte pieces
    (79, "float16", "e8m0", 1, 0),     # odd rows (2-byte token vectors): separate pass
])
def test_scale_paths(h, tok, scales, S, inline):
    dev = _dev()
    w = workloads.random_case(h + S, 6, 5, h, tokens_dtype=tok, count_range=(0, 40), scales=scales, S=S,
                              weight=True, idx_type=h % 2)
    t = workloads.torch_inputs(w, dev)
    call, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"], expert_topk_weight=t["weight"],
                            idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"])
    assert call.plan()["scale_inline_bytes"] == inline
    check(w)
    check(w, phases=True)


def test_sparse_cells_window_fallback():
    """Rows whose cells lie more than 64 cells apart inside one 64-row batch."""
    counts = np.zeros((40, 100), np.int64)
    counts[0, 0] = 3
    counts[39, 99] = 70
    counts[20, 50] = 1
    a = int(counts.sum())
    rng = np.random.default_rng(5)
    w = workloads.Workload("sparse", counts, rng.integers(0, 256, (a, 16), dtype=np.uint8), "int8", 16,
                           idx_type=1)
    check(w)


def test_repeat_calls_identical():
    dev = _dev()
    w = workloads.random_case(99, 8, 8, 512, tokens_dtype="int8", scales="e8m0", weight=True)
    first, _ = run_hip(w, dev)
    second, _ = run_hip(w, dev)
    for x, y in zip(first, second):
        assert np.array_equal(x, y)


# --- device-detected count errors -------------------------------------------

@pytest.mark.parametrize("phases", [False, True], ids=["whole", "phases"])
@pytest.mark.parametrize("kind", ["negative", "sum_low", "sum_high", "too_large"])
def test_bad_counts_write_nothing(kind, phases):
    dev = _dev()
    rng = np.random.default_rng(3)
    counts = rng.integers(1, 5, (4, 3)).astype(np.int64)
    a = int(counts.sum())
    if kind == "negative":
        counts[1, 1] = -counts[1, 1]
        counts[2, 2] += 2 * abs(counts[1, 1])    # keep the sum at a
    elif kind == "sum_low":
        counts[0, 0] -= 1
    elif kind == "sum_high":
        counts[0, 0] += 1
    else:
        counts[3, 2] = (1 << 32) + counts[3, 2]  # above INT32_MAX
    tok = rng.integers(0, 256, (a, 64), dtype=np.uint8)
    w = workloads.Workload(f"bad_{kind}", counts, tok, "int8", 64,
                           rng.standard_normal(a, dtype=np.float32), "float32",
                           rng.random((a, 1), dtype=np.float32), 1, 0)
    out, status = run_hip(w, dev, phases=phases)
    assert status == _lib.ERROR_BAD_COUNTS
    for o in out:
        assert (o == SENTINEL).all(), kind


def test_bad_counts_large_table():
    """A count matrix too large for the single-kernel path, with a bad sum."""
    dev = _dev()
    rng = np.random.default_rng(9)
    counts = rng.integers(0, 3, (256, 64)).astype(np.int32)
    a = int(counts.sum())
    counts[100, 7] += 1
    w = workloads.Workload("bad_large", counts, rng.integers(0, 256, (a, 32), dtype=np.uint8), "int8", 32)
    out, status = run_hip(w, dev)
    assert status == _lib.ERROR_BAD_COUNTS
    for o in out:
        assert (o == SENTINEL).all()


def test_bad_counts_raise_with_check():
    dev = _dev()
    counts = torch.tensor([[2, 1], [1, 1]], dtype=torch.int32, device=dev)
    tokens = torch.zeros((4, 8), dtype=torch.float16, device=dev)   # sum is 5, A is 4
    with pytest.raises(ValueError):
        api.moe_re_routing(tokens, counts, check=True)


@pytest.mark.parametrize("first", ["offsets", "fused_call", "one_launch_call"])
def test_gather_needs_matching_tables(first):
    """A gather phase on a workspace whose table was built for another
    (A, N, E), or that holds no table (a whole call in one launch, fused or
    one-launch stream kernel, builds none), writes nothing."""
    dev = _dev()
    h = 1024 if first == "one_launch_call" else 64
    w1 = workloads.random_case(1, 3, 3, h, tokens_dtype="int8", count_range=(1, 5))
    t1 = workloads.torch_inputs(w1, dev)
    call1, _ = api.make_call(t1["tokens"], t1["counts"])
    if first == "offsets":
        call1.run_offsets()
    else:
        assert call1.plan()["fused"] == (2 if first == "one_launch_call" else 1)
        call1.run()
    w2 = (workloads.random_case(2, 3, 4, h, tokens_dtype="int8", count_range=(1, 5)) if first == "offsets"
          else w1)
    t2 = workloads.torch_inputs(w2, dev)
    args, outs = api.prepare(t2["tokens"], t2["counts"])
    for o in outs:
        if o.numel():
            o.view(-1).view(torch.uint8).fill_(SENTINEL)
    call2, outs = api.make_call(t2["tokens"], t2["counts"], out=outs, workspace=call1.workspace)
    call2.run_gather()
    torch.cuda.synchronize()
    for o in (outs[0], outs[2]):
        assert (_bytes(o) == SENTINEL).all()


def test_python_api_shapes():
    dev = _dev()
    w = workloads.make("tiny")
    t = workloads.torch_inputs(w, dev)
    p_tok, p_sc, p_idx, p_etn, p_w = api.moe_re_routing(t["tokens"], t["counts"], per_token_scales=t["scales"],
                                                        check=True)
    assert p_tok.shape == t["tokens"].shape and p_tok.dtype == t["tokens"].dtype
    assert p_sc.shape == (w.A,) and p_sc.dtype == torch.float32
    assert p_idx.shape == (w.A,) and p_idx.dtype == torch.int32
    assert p_etn.shape == (w.E,) and p_etn.dtype == t["counts"].dtype
    assert p_w.shape == (0,) and p_w.dtype == torch.float32
    ref = run_oracle(w)
    assert np.array_equal(p_idx.cpu().numpy(), ref[2])
