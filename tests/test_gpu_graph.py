"""The whole call captured in a HIP graph (torch.cuda.CUDAGraph on a side
stream) and replayed: the launch path makes no allocation, no memset and no
synchronization, so a captured call is the same kernels with the same
pointers. Each replay follows eager work that rewrites the inputs in place
and a synchronization, and is checked byte for byte against the oracle on
those inputs (a replay that reused stale data would fail)."""
import numpy as np
import pytest
import torch

from gpu_helpers import _dev, assert_parity, run_oracle
from moe_token_re_amd import _lib, api, workloads

pytestmark = pytest.mark.gpu


def _host_bytes(outs):
    return [o.contiguous().view(-1).view(torch.uint8).cpu().numpy() for o in outs]


@pytest.mark.parametrize("direction", [_lib.FORWARD, _lib.INVERSE], ids=["forward", "inverse"])
# (N, E, H, counts, the plan's launch): the fused kernel, the two kernels, and
# the one-launch stream kernel (50 MiB of 1 KiB bf16 rows; 384 cells: eight a
# lane; 158-byte rows: its byte form)
@pytest.mark.parametrize("n,e,h,count_range,fused", [(4, 3, 256, (0, 6), 1), (40, 30, 256, (0, 6), 0),
                                                     (16, 16, 512, (180, 221), 2), (16, 24, 512, (60, 100), 2),
                                                     (16, 16, 79, (180, 221), 2)],
                         ids=["fused", "two_kernel", "one_launch", "one_launch_384", "one_launch_bytes"])
def test_graph_replays_match_oracle(n, e, h, count_range, fused, direction):
    dev = _dev()
    base = workloads.random_case(71, n, e, h, tokens_dtype="bfloat16", count_range=count_range, scales="as", S=3,
                                 weight=True, idx_type=1, etn_type=0)
    t = workloads.torch_inputs(base, dev)
    side = torch.cuda.Stream(dev)
    call, outs = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"],
                               expert_topk_weight=t["weight"], expert_token_num_type=base.etn_type,
                               idx_type=base.idx_type, stream=side, direction=direction)
    assert call.plan()["fused"] == fused
    with torch.cuda.stream(side):
        call.run()  # eager first call: one-time per-device set-up happens outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for replay in range(4):
        # new token rows, scales and weights of the same shapes, written eagerly in place
        # (the captured call keeps its count matrix; A is fixed by the shapes)
        w = workloads.Workload(f"graph_replay_{replay}", base.counts,
                               rng.integers(0, 256, base.tokens.nbytes, dtype=np.uint8)
                               .view(base.tokens.dtype).reshape(base.tokens.shape),
                               base.tokens_dtype, base.H,
                               rng.standard_normal(base.scales.shape, dtype=np.float32), base.scales_dtype,
                               rng.random(base.weight.shape, dtype=np.float32), base.etn_type, base.idx_type)
        fresh = workloads.torch_inputs(w, dev)
        for key in ("tokens", "scales", "weight"):
            t[key].copy_(fresh[key])
        for o in outs:
            if o.numel():
                o.view(-1).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert call.device_status() == _lib.SUCCESS
        assert_parity(w, _host_bytes(outs), run_oracle(w, direction))
