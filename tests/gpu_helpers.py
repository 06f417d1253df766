"""Shared by the GPU parity tests: run the HIP path through the C ABI on a
workload (outputs pre-filled with a sentinel) and compare it with the CPU
oracle byte for byte, in either direction.

Every output, and the workspace, lies between two guard bands of GUARD
sentinel bytes inside a larger buffer; after each call the guards must be
untouched, so a write before or past the end of any buffer fails the test."""
import numpy as np
import pytest
import torch

from moe_token_re_amd import _lib, api, workloads
from oracle import oracle

SENTINEL = 0xA5
GUARD = 4096  # sentinel bytes before and after each guarded buffer (keeps 256-byte alignment)


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bytes(t):
    return t.contiguous().view(-1).view(torch.uint8).cpu().numpy()


def _np_bytes(a):
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


class Guarded:
    """Tensors of given shapes and dtypes, each the middle of a sentinel-filled
    uint8 buffer with GUARD bytes on either side."""

    def __init__(self):
        self._bufs = []  # (name, buffer, payload bytes)

    def like(self, name, t):
        if t.numel() == 0:
            return t
        nbytes = t.numel() * t.element_size()
        buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=t.device)
        self._bufs.append((name, buf, nbytes))
        return buf[GUARD:GUARD + nbytes].view(t.dtype).view(t.shape)

    def bytes(self, name, nbytes, device):
        buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=device)
        self._bufs.append((name, buf, nbytes))
        return buf[GUARD:GUARD + nbytes]

    def check(self, where=""):
        """Asserts that no guard byte changed (call after synchronizing)."""
        for name, buf, nbytes in self._bufs:
            b = buf.cpu().numpy()
            head, tail = b[:GUARD], b[GUARD + nbytes:]
            assert (head == SENTINEL).all(), f"{where}: write before {name} (guard byte {np.flatnonzero(head != SENTINEL)[:4]})"
            assert (tail == SENTINEL).all(), f"{where}: write past the end of {name} (+{np.flatnonzero(tail != SENTINEL)[:4]})"


OUT_NAMES = ("permute_tokens", "permute_per_token_scales", "permute_token_idx", "expert_token_num",
             "permute_topk_weight")


def guarded_call(t, dev, guards, **kw):
    """make_call with every output and the workspace inside guard bands, the
    outputs pre-filled with the sentinel."""
    _, outs = api.prepare(t["tokens"], t["counts"], **kw)
    outs = tuple(guards.like(n, o) for n, o in zip(OUT_NAMES, outs))
    for o in outs:
        if o.numel():
            o.view(-1).view(torch.uint8).fill_(SENTINEL)
    A, N, E = t["tokens"].shape[0], t["counts"].shape[0], t["counts"].shape[1]
    ws = guards.bytes("workspace", api.workspace_size(A, N, E), dev)
    return api.make_call(t["tokens"], t["counts"], out=outs, workspace=ws, **kw)


def run_hip(w: workloads.Workload, dev, phases=False, direction=_lib.FORWARD):
    """Runs the HIP path on a workload with outputs pre-filled with a sentinel,
    inside guard bands. Returns (outputs on the host as raw bytes, the device
    status code); fails if any guard byte changed."""
    print(f"[hip] {w.name} dir={direction} A={w.A} H={w.H} N={w.N} E={w.E} tok={w.tokens_dtype} "
          f"scales={w.scales_dtype} w={w.weight is not None} etn={w.etn_type} idx={w.idx_type}", flush=True)
    t = workloads.torch_inputs(w, dev)
    kw = dict(per_token_scales=t["scales"], expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
              idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"], direction=direction)
    guards = Guarded()
    call, outs = guarded_call(t, dev, guards, **kw)
    if phases:
        call.run_offsets()
        call.run_gather()
    else:
        call.run()
    status = call.device_status()
    torch.cuda.synchronize()
    guards.check(w.name)
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
