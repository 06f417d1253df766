"""Parity at millions of rows, byte for byte against the CPU oracle, through
the C ABI: grids of millions of 64-lane gather workgroups, row maps of
several MiB, offsets kernels with thousands of workgroups (one per 256 rows)
and banded offsets with the largest workgroup split (16 per band, each
walking ~100k source rows), in both directions, with every per-row item
(scales of each layout, weights, both index forms). The one-launch kernel at
its largest grid (2^26 - 1 workgroups, 68 GB of token rows) is checked in
full against the oracle's offsets."""
import numpy as np
import pytest
import torch

from gpu_helpers import _dev, check
from moe_token_re_amd import _lib, api, workloads
from oracle import oracle

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


# The largest call the one-launch kernel takes with 1040-byte rows: its grid of
# 67,108,863 workgroups (item waves plus one per KiB of the input rows) is the
# most a launch of 64-lane workgroups holds; one row more takes two kernels.
# 4,278,511,315 token vectors: the 32-bit vector numbers come within 2^24 of
# their limit.
LARGEST_A, LARGEST_H = 65_823_251, 1040


@pytest.mark.parametrize("direction", [_lib.FORWARD, _lib.INVERSE], ids=["forward", "inverse"])
def test_one_launch_largest_grid(direction):
    dev = _dev()
    if torch.cuda.get_device_properties(dev).total_memory < 200 * (1 << 30):
        pytest.skip("needs about 140 GB of device memory")
    A, H = LARGEST_A, LARGEST_H
    rng = np.random.default_rng(104)
    cuts = np.sort(rng.choice(np.arange(1, A), 15, replace=False))
    counts = np.diff(np.concatenate([[0], cuts, [A]])).astype(np.int32).reshape(4, 4)
    counts[1, 2] += counts[0, 3]  # two empty cells, the sum kept
    counts[0, 3] = 0
    counts[3, 0] += counts[2, 1]
    counts[2, 1] = 0
    assert int(counts.sum()) == A
    tokens = torch.empty((A, H), dtype=torch.int8, device=dev)
    tokens.random_(-128, 128)
    scales = torch.randn(A, device=dev)
    weight = torch.rand((A, 1), device=dev)
    call, outs = api.make_call(tokens, torch.from_numpy(counts).to(dev), per_token_scales=scales,
                               expert_topk_weight=weight, direction=direction)
    plan = call.plan()
    assert plan["fused"] == 2 and plan["one_launch_workgroups"] == (1 << 26) - 1, plan
    print(f"[largest] A={A} H={H} direction={direction} plan={plan}", flush=True)
    call.run()
    assert call.device_status() == _lib.SUCCESS
    out_tokens, out_scales, idx, etn, out_weight = outs
    # the input row of every output row, from the oracle's offsets (forward:
    # output rows DstOffset + k take input rows SrcOffset + k; inverse: the reverse)
    src_off, dst_off = (x.reshape(-1) for x in oracle.offsets(counts))
    expect = torch.empty(A, dtype=torch.int64, device=dev)
    for m, c in enumerate(counts.reshape(-1).tolist()):
        s, d = int(src_off[m]), int(dst_off[m])
        out0, in0 = (d, s) if direction == _lib.FORWARD else (s, d)
        expect[out0:out0 + c] = torch.arange(in0, in0 + c, device=dev)
    assert torch.equal(idx.long(), expect)
    assert torch.equal(etn.cpu(), torch.from_numpy(counts.sum(0).astype(np.int32)))
    assert torch.equal(out_scales.view(torch.int32), scales.view(torch.int32)[expect])
    assert torch.equal(out_weight.view(torch.int32), weight.view(torch.int32)[expect])
    step = 1 << 21
    for r0 in range(0, A, step):
        r1 = min(A, r0 + step)
        assert torch.equal(out_tokens[r0:r1], tokens.index_select(0, expect[r0:r1])), (r0, r1)
    del tokens, scales, weight, outs, out_tokens, out_scales, idx, etn, out_weight, expect, call
    torch.cuda.empty_cache()
