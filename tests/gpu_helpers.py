"""Shared by the GPU parity tests: run the HIP path through the C ABI on a
workload (outputs pre-filled with a sentinel) and compare it with the CPU
oracle byte for byte, in either direction."""
import numpy as np
import pytest
import torch

from moe_token_re_amd import _lib, api, workloads
from oracle import oracle

SENTINEL = 0xA5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bytes(t):
    return t.contiguous().view(-1).view(torch.uint8).cpu().numpy()


def _np_bytes(a):
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def run_hip(w: workloads.Workload, dev, phases=False, direction=_lib.FORWARD):
    """Runs the HIP path on a workload with outputs pre-filled with a sentinel.
    Returns (outputs on the host as raw bytes, the device status code)."""
    print(f"[hip] {w.name} dir={direction} A={w.A} H={w.H} N={w.N} E={w.E} tok={w.tokens_dtype} "
          f"scales={w.scales_dtype} w={w.weight is not None} etn={w.etn_type} idx={w.idx_type}", flush=True)
    t = workloads.torch_inputs(w, dev)
    kw = dict(per_token_scales=t["scales"], expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
              idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"], direction=direction)
    args, outs = api.prepare(t["tokens"], t["counts"], **kw)
    for o in outs:
        if o.numel():
            o.view(-1).view(torch.uint8).fill_(SENTINEL)
    call, outs = api.make_call(t["tokens"], t["counts"], out=outs, **kw)
    if phases:
        call.run_offsets()
        call.run_gather()
    else:
        call.run()
    status = call.device_status()
    torch.cuda.synchronize()
    return [_bytes(o) for o in outs], status


def run_oracle(w: workloads.Workload, direction=_lib.FORWARD):
    fn = oracle.reroute if direction == _lib.FORWARD else oracle.reroute_inverse
    return fn(w.tokens, w.counts, w.scales, w.weight, w.etn_type, w.idx_type)


def assert_parity(w, hip_out, ref):
    p_tok, p_sc, p_idx, p_etn, p_w = hip_out
    r_tok, r_sc, r_idx, r_etn, r_w = ref
    assert np.array_equal(p_tok, _np_bytes(r_tok)), f"{w.name}: permute_tokens differ"
    assert np.array_equal(p_idx.view(np.int32), r_idx), f"{w.name}: permute_token_idx differ"
    assert np.array_equal(p_etn, _np_bytes(r_etn)), f"{w.name}: expert_token_num differ"
    if w.scales is not None:
        assert np.array_equal(p_sc, _np_bytes(r_sc)), f"{w.name}: permute_per_token_scales differ"
    if w.weight is not None:
        assert np.array_equal(p_w, _np_bytes(r_w)), f"{w.name}: permute_topk_weight differ"


def check(w, phases=False, direction=_lib.FORWARD):
    dev = _dev()
    hip_out, status = run_hip(w, dev, phases, direction)
    assert status == _lib.SUCCESS, _lib.status_string(status)
    assert_parity(w, hip_out, run_oracle(w, direction))
