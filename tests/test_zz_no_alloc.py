"""moe_rerouting_v2_noalloc, the entry point for callers that cannot allocate
(no workspace argument: the library's static device scratch), against
moe_rerouting_v2 with a workspace of its own, through the C ABI on the GPU.

Seven calls go out back to back on one stream, each with a smaller input than
the one before, so each finds the scratch holding the previous call's header
and row map: a 2-million-row call that fills the scratch nearly to its limit,
the 256 x 64 banded shape, two calls of the one-launch kernel (384 and 256
cells), a 32 x 32 call with 158-byte rows, a 16 x 16 call with 158-byte rows
(the one-launch kernel's byte form), and the single-kernel tiny call. Every
output byte must equal the existing entry point's on the same inputs (and the
oracle's)."""
import numpy as np
import pytest
import torch

from gpu_helpers import SENTINEL, Guarded, _bytes, _dev, assert_parity, guarded_call, run_oracle
from moe_token_re_amd import _lib, api, workloads

pytestmark = pytest.mark.gpu


def _cases():
    return [
        # 16 x 16 counts of about 7800 rows each: the row map nearly fills the scratch
        workloads.random_case(71, 16, 16, 16, tokens_dtype="float16", count_range=(7000, 8600), scales="a",
                              weight=True),
        workloads.make("tiny_segments"),
        # one-launch kernel: 16 x 24 counts (eight cells a lane), then 16 x 16 (four a lane)
        workloads.random_case(73, 16, 24, 1024, tokens_dtype="int8", count_range=(60, 100), scales="a",
                              weight=True),
        workloads.random_case(74, 16, 16, 1024, tokens_dtype="bfloat16", count_range=(40, 60), scales="e8m0",
                              idx_type=1, counts_dtype=np.int64),
        workloads.random_case(72, 32, 32, 79, tokens_dtype="float16", count_range=(0, 20), scales="e8m0",
                              idx_type=1, etn_type=0),
        workloads.random_case(75, 16, 16, 79, tokens_dtype="float16", count_range=(15, 25), scales="a",
                              weight=True),
        workloads.make("tiny"),
    ]


def _prepared(w, dev, guards):
    """Inputs on the GPU, and a prepared call whose outputs lie inside guard
    bands, pre-filled with the sentinel."""
    t = workloads.torch_inputs(w, dev)
    kw = dict(per_token_scales=t["scales"], expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
              idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"])
    call, outs = guarded_call(t, dev, guards, **kw)
    return t, call, outs


def test_noalloc_matches_workspace_entry_point():
    dev = _dev()
    cases = _cases()
    sizes = [_lib.load().mrr_workspace_size(w.A, w.N, w.E) for w in cases]
    assert all(s <= _lib.NOALLOC_SCRATCH_BYTES for s in sizes), sizes
    assert sizes[0] > _lib.NOALLOC_SCRATCH_BYTES * 9 // 10, sizes
    assert [w.A for w in cases] == sorted((w.A for w in cases), reverse=True)
    guards = Guarded()
    noalloc = [_prepared(w, dev, guards) for w in cases]
    torch.cuda.synchronize()
    for w, (_, call, _) in zip(cases, noalloc):  # back to back, one stream, no wait in between
        print(f"[noalloc] {w.name} A={w.A} N={w.N} E={w.E} H={w.H} plan={call.plan()}", flush=True)
        call.run_noalloc()
    torch.cuda.synchronize()
    guards.check("noalloc calls")
    for w, (_, _, outs) in zip(cases, noalloc):
        _, ref_call, ref_outs = _prepared(w, dev, Guarded())
        ref_call.run()
        assert ref_call.device_status() == _lib.SUCCESS
        torch.cuda.synchronize()
        got = [_bytes(o) for o in outs]
        want = [_bytes(o) for o in ref_outs]
        for k, (g, r) in enumerate(zip(got, want)):
            if k == 1 and w.scales is None:
                continue  # permute_per_token_scales has no defined value without scales
            if k == 4 and w.weight is None:
                continue
            assert np.array_equal(g, r), (w.name, k)
        assert_parity(w, got, run_oracle(w))


def test_noalloc_repeat_and_rejects_too_large():
    """The same call twice gives the same bytes; a call whose workspace would
    exceed the scratch is refused before any launch and writes nothing."""
    dev = _dev()
    w = workloads.make("tiny_segments")
    guards = Guarded()
    _, call, outs = _prepared(w, dev, guards)
    call.run_noalloc()
    torch.cuda.synchronize()
    first = [_bytes(o) for o in outs]
    call.run_noalloc()
    torch.cuda.synchronize()
    assert all(np.array_equal(a, b) for a, b in zip(first, [_bytes(o) for o in outs]))
    big = workloads.random_case(73, 16, 16, 16, count_range=(8300, 8400))
    assert _lib.load().mrr_workspace_size(big.A, big.N, big.E) > _lib.NOALLOC_SCRATCH_BYTES
    _, bcall, bouts = _prepared(big, dev, guards)
    with pytest.raises(api.MrrValueError):
        bcall.run_noalloc()
    torch.cuda.synchronize()
    assert all((_bytes(o) == SENTINEL).all() for o in bouts if o.numel())
    guards.check("noalloc repeat")
