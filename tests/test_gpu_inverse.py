"""Parity of the inverse re-route (expert-major rows back to rank-major order,
mrr_args.direction = MRR_INVERSE) with the CPU oracle's inverse, byte for byte,
through the C ABI: the named workloads at full size (whole call and the two
phases), every offsets kernel (fused, single workgroup with one cell or
chunks per thread, banded, through global memory), a seeded fuzz, round trips
through the forward call, and tables built for the other direction."""
import numpy as np
import pytest
import torch

from gpu_helpers import SENTINEL, _bytes, _dev, check, run_hip
from moe_token_re_amd import _lib, api, workloads

pytestmark = pytest.mark.gpu

INV = _lib.INVERSE


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_inverse_named_workload_full_size(name):
    check(workloads.make(name), direction=INV)


@pytest.mark.parametrize("name", ["pages_shape", "tiny_segments", "tiny"])
def test_inverse_two_phases(name):
    check(workloads.make(name), phases=True, direction=INV)


# One shape per offsets kernel: fused (M <= 256), one cell per thread, chunks
# of 3 and 17 (more than 1024 experts), banded, and through global memory.
@pytest.mark.parametrize("n,e", [(6, 5), (32, 32), (2, 1025), (16, 1088), (33, 32), (256, 64), (97, 96),
                                 (17, 1025), (520, 256)])
def test_inverse_offsets_kernels(n, e):
    w = workloads.random_case(n * 3 + e, n, e, 40, tokens_dtype="int8", count_range=(0, 4), weight=True,
                              scales="a", idx_type=(n + e) % 2, etn_type=(n * e) % 2)
    check(w, direction=INV)
    check(w, phases=True, direction=INV)


def _fuzz_cases():
    rng = np.random.default_rng(77)
    kinds = ["float16", "bfloat16", "int8", "float8_e4m3fn", "hifloat8", "float4_e2m1fn_x2"]
    out = []
    for k in range(16):
        tok = kinds[k % len(kinds)]
        h = int(rng.choice([2, 64, 79, 130, 2048, 7168]))
        if tok.startswith("float4") and h % 2:
            h += 1
        n, e = [(4, 2), (16, 16), (7, 13), (1, 9), (33, 5), (3, 1)][k % 6]
        out.append(dict(seed=5000 + k, N=n, E=e, H=h, tokens_dtype=tok,
                        counts_dtype=np.int64 if k % 3 == 0 else np.int32,
                        count_range=(0, 9) if k % 2 else (1, 30), scales=[None, "a", "as", "e8m0"][k % 4],
                        S=int(rng.integers(1, 20)), weight=bool(k % 4 != 0), etn_type=k % 2,
                        idx_type=(k // 2) % 2))
    return out


@pytest.mark.parametrize("case", _fuzz_cases(), ids=lambda c: f"s{c['seed']}")
def test_inverse_fuzz(case):
    w = workloads.random_case(**case)
    check(w, direction=INV)
    check(w, phases=True, direction=INV)


@pytest.mark.parametrize("name", ["pages_shape", "mxfp8_skewed", "tiny_segments"])
def test_round_trip_full_size(name):
    """Forward then inverse on the GPU gives back the input bytes, and the
    inverse's gather index is the forward's scatter index."""
    dev = _dev()
    w = workloads.make(name)
    t = workloads.torch_inputs(w, dev)
    kw = dict(expert_token_num_type=w.etn_type, tokens_dtype=t["tokens_dtype"])
    f_tok, f_sc, f_idx, _, f_w = api.moe_re_routing(t["tokens"], t["counts"], per_token_scales=t["scales"],
                                                    expert_topk_weight=t["weight"], idx_type=1, check=True, **kw)
    b_tok, b_sc, b_idx, _, b_w = api.moe_re_routing_inverse(
        f_tok, t["counts"], per_token_scales=t["scales"] if t["scales"] is None else f_sc,
        expert_topk_weight=t["weight"] if t["weight"] is None else f_w, idx_type=0, check=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(_u8(b_tok), _u8(t["tokens"]))
    if t["scales"] is not None:
        assert torch.equal(_u8(b_sc), _u8(t["scales"]))
    if t["weight"] is not None:
        assert torch.equal(_u8(b_w), _u8(t["weight"]))
    assert torch.equal(b_idx, f_idx)


def _u8(x):
    return x.contiguous().view(-1).view(torch.uint8)


@pytest.mark.parametrize("first_dir", [_lib.FORWARD, INV])
def test_gather_rejects_table_of_other_direction(first_dir):
    """A gather phase on a workspace whose table was built for the other
    direction (same counts, same shapes) writes nothing."""
    dev = _dev()
    w = workloads.random_case(9, 40, 30, 64, tokens_dtype="int8", count_range=(1, 4))
    t = workloads.torch_inputs(w, dev)
    call1, _ = api.make_call(t["tokens"], t["counts"], direction=first_dir)
    call1.run_offsets()
    other = INV if first_dir == _lib.FORWARD else _lib.FORWARD
    args, outs = api.prepare(t["tokens"], t["counts"], direction=other)
    for o in outs:
        if o.numel():
            o.view(-1).view(torch.uint8).fill_(SENTINEL)
    call2, outs = api.make_call(t["tokens"], t["counts"], out=outs, workspace=call1.workspace, direction=other)
    call2.run_gather()
    torch.cuda.synchronize()
    for o in (outs[0], outs[2]):
        assert (_bytes(o) == SENTINEL).all()


def test_inverse_bad_counts_write_nothing():
    dev = _dev()
    rng = np.random.default_rng(8)
    for n, e in ((4, 3), (256, 64)):
        counts = rng.integers(1, 4, (n, e)).astype(np.int32)
        a = int(counts.sum())
        counts[n - 1, 0] = -1
        w = workloads.Workload(f"inv_bad_{n}x{e}", counts, rng.integers(0, 256, (a, 8), dtype=np.uint8), "int8", 8)
        for phases in (False, True):
            out, status = run_hip(w, dev, phases=phases, direction=INV)
            assert status == _lib.ERROR_BAD_COUNTS
            for o in out:
                assert (o == SENTINEL).all()
