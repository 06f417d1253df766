"""Python binding of the MoE re-routing operator (MoeReRoutingV2) on MI355X.

Argument marshalling only: torch provides device memory and the stream; every
step of the operator runs in the HIP kernels of libmoe_rerouting_v2.so. The
signature mirrors the operator's Torch API (page "CANN ops-transformer
MoeReRoutingV2", nlpx.cn, section "PyTorch API 调用"), plus the `tokens_dtype`
tag of its Torch front end for uint8-stored hifloat8 / fp4 tokens, and output
shapes follow its InferShape rules:
  permute_tokens            tokens' shape and dtype
  permute_per_token_scales  scales' shape and dtype; [A] float32 (meaningless,
                            never written) when the scales are absent
  permute_token_idx         [A] int32
  expert_token_num          [E], counts' dtype
  permute_topk_weight       weight's shape; an empty (0,) float32 when absent
moe_re_routing_inverse() runs the same moves backwards (expert-major rows back
to rank-major order; the article's formulas read in reverse), with the same
arguments and output shapes.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_TOKEN_DTYPES = {
    torch.float16: _lib.F16,
    torch.bfloat16: _lib.BF16,
    torch.int8: _lib.I8,
    torch.float8_e5m2: _lib.F8_E5M2,
    torch.float8_e4m3fn: _lib.F8_E4M3FN,
    torch.float4_e2m1fn_x2: _lib.F4_E2M1,
}
# uint8 storage tagged with the real element type (Torch front end's tokens_dtype)
_TAGGED = {
    "hifloat8": _lib.HIF8,
    "float4_e2m1fn_x2": _lib.F4_E2M1,
    "float4_e1m2fn_x2": _lib.F4_E1M2,
    "float8_e5m2": _lib.F8_E5M2,
    "float8_e4m3fn": _lib.F8_E4M3FN,
    "int8": _lib.I8,
}
_FP4 = (_lib.F4_E2M1, _lib.F4_E1M2)


class MrrError(Exception):
    """A non-success status from the library; `status` holds the code."""

    def __init__(self, status: int, where: str = ""):
        self.status = status
        super().__init__(f"{where}: {_lib.status_string(status)}" if where else _lib.status_string(status))


class MrrValueError(MrrError, ValueError):
    pass


class MrrTypeError(MrrError, TypeError):
    pass


class MrrRuntimeError(MrrError, RuntimeError):
    pass


def _raise(status: int, where: str):
    if status == _lib.ERROR_UNSUPPORTED_DTYPE:
        raise MrrTypeError(status, where)
    if status == _lib.ERROR_HIP:
        raise MrrRuntimeError(status, where)
    raise MrrValueError(status, where)


def workspace_size(A: int, N: int, E: int) -> int:
    """Bytes of workspace a call with A rows and an N x E count matrix needs."""
    return int(_lib.load().mrr_workspace_size(A, N, E))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prepare(tokens, expert_token_num_per_rank, *, per_token_scales=None, expert_topk_weight=None,
            expert_token_num_type=1, idx_type=0, tokens_dtype=None, out=None, direction=_lib.FORWARD):
    """Checks the tensors' dtypes and ranks, allocates the outputs (or takes
    `out`, a 5-tuple like the result) and fills an MrrArgs. Returns (args, outputs)."""
    dev = tokens.device
    if dev.type != "cuda":
        raise ValueError("tokens must be on a GPU device (there is no CPU path)")
    _check_tensor("tokens", tokens, dev)
    _check_tensor("expert_token_num_per_rank", expert_token_num_per_rank, dev)
    if tokens.dim() != 2 or expert_token_num_per_rank.dim() != 2:
        raise ValueError("tokens and expert_token_num_per_rank must be 2-D")
    if tokens_dtype is not None:
        if tokens.dtype not in (torch.uint8, torch.int8) or tokens_dtype not in _TAGGED:
            raise TypeError(f"tokens_dtype={tokens_dtype!r} needs uint8 storage and one of {sorted(_TAGGED)}")
        tdt = _TAGGED[tokens_dtype]
    elif tokens.dtype in _TOKEN_DTYPES:
        tdt = _TOKEN_DTYPES[tokens.dtype]
    else:
        raise TypeError(f"unsupported tokens dtype {tokens.dtype}")
    counts = expert_token_num_per_rank
    if counts.dtype == torch.int32:
        cdt = _lib.I32
    elif counts.dtype == torch.int64:
        cdt = _lib.I64
    else:
        raise TypeError(f"expert_token_num_per_rank must be int32 or int64, got {counts.dtype}")
    A = tokens.shape[0]
    H = tokens.shape[1] * (2 if tdt in _FP4 else 1)
    N, E = counts.shape

    a = _lib.MrrArgs()
    a.tokens = _ptr(tokens)
    a.tokens_dtype = tdt
    a.A, a.H = A, H
    a.expert_token_num_per_rank = _ptr(counts)
    a.counts_dtype = cdt
    a.N, a.E = N, E
    if per_token_scales is not None:
        s = per_token_scales
        _check_tensor("per_token_scales", s, dev)
        if s.dtype == torch.float32:
            a.scales_dtype = _lib.F32
        elif s.dtype in (torch.float8_e8m0fnu, torch.uint8):
            a.scales_dtype = _lib.F8_E8M0
        else:
            raise TypeError(f"unsupported per_token_scales dtype {s.dtype}")
        if s.dim() > 3:
            raise ValueError("per_token_scales must be 1-, 2- or 3-D")
        a.per_token_scales = _ptr(s)
        a.scales_ndim = s.dim()
        for k in range(s.dim()):
            a.scales_dims[k] = s.shape[k]
    if expert_topk_weight is not None:
        w = expert_topk_weight
        _check_tensor("expert_topk_weight", w, dev)
        if w.dtype != torch.float32:
            raise TypeError("expert_topk_weight must be float32")
        if w.dim() != 2 or w.shape[0] != A or w.shape[1] != 1:
            raise ValueError("expert_topk_weight must be 2-D [A, 1]")
        a.expert_topk_weight = _ptr(w)

    # the outputs as InferShape gives them: (dtype, element count) each
    sc, w = per_token_scales, expert_topk_weight
    want = (("permute_tokens", tokens.dtype, tokens.numel()),
            ("permute_per_token_scales", sc.dtype if sc is not None else torch.float32,
             sc.numel() if sc is not None else A),
            ("permute_token_idx", torch.int32, A),
            ("expert_token_num", counts.dtype, E),
            ("permute_topk_weight", torch.float32, w.numel() if w is not None else 0))
    if out is None:
        p_tok = torch.empty_like(tokens)
        p_sc = (torch.empty_like(per_token_scales) if per_token_scales is not None
                else torch.empty((A,), dtype=torch.float32, device=dev))
        p_idx = torch.empty((A,), dtype=torch.int32, device=dev)
        p_etn = torch.empty((E,), dtype=counts.dtype, device=dev)
        p_w = (torch.empty_like(expert_topk_weight) if expert_topk_weight is not None
               else torch.empty((0,), dtype=torch.float32, device=dev))
        out = (p_tok, p_sc, p_idx, p_etn, p_w)
    else:
        # The library sees only pointers: every output it writes must hold
        # exactly the bytes InferShape gives it, densely, on this device.
        if not isinstance(out, (tuple, list)) or len(out) != 5:
            raise ValueError("out must be a 5-tuple like the result")
        for t, (name, dtype, numel) in zip(out, want):
            if name == "permute_per_token_scales" and per_token_scales is None:
                continue  # never written when the scales are absent
            if name == "permute_topk_weight" and expert_topk_weight is None:
                continue  # never written when the weight is absent
            _check_tensor(name, t, dev)
            if t.dtype != dtype:
                raise TypeError(f"out {name} has dtype {t.dtype}, expected {dtype}")
            if t.numel() != numel:
                raise ValueError(f"out {name} has {t.numel()} elements, expected {numel}")
    p_tok, p_sc, p_idx, p_etn, p_w = out
    a.permute_tokens = _ptr(p_tok)
    a.permute_per_token_scales = _ptr(p_sc) if per_token_scales is not None else None
    a.permute_token_idx = _ptr(p_idx)
    a.expert_token_num = _ptr(p_etn)
    a.permute_topk_weight = _ptr(p_w) if expert_topk_weight is not None else None
    a.expert_token_num_type = int(expert_token_num_type)
    a.idx_type = int(idx_type)
    a.direction = int(direction)
    return a, out


class PreparedCall:
    """One set of arguments, workspace and stream, callable repeatedly with low
    host overhead (no re-marshalling): run(), or the two phases alone."""

    def __init__(self, args: _lib.MrrArgs, workspace: torch.Tensor, stream: torch.cuda.Stream, keep=()):
        self.args = args
        self.workspace = workspace
        self.stream = stream
        self._keep = keep  # tensors the pointers in args refer to
        self._lib = _lib.load()
        self._pargs = ctypes.byref(args)
        self._ws = workspace.data_ptr()
        self._wsb = workspace.numel() * workspace.element_size()
        self._s = stream.cuda_stream

    def validate(self) -> int:
        return self._lib.mrr_validate(self._pargs, self._ws, self._wsb)

    def plan(self) -> dict:
        """How moe_rerouting_v2 launches this call (mrr_describe_plan)."""
        info = _lib.MrrPlanInfo()
        st = self._lib.mrr_describe_plan(self._pargs, self._ws, self._wsb, ctypes.byref(info))
        if st != _lib.SUCCESS:
            _raise(st, "mrr_describe_plan")
        return {name: getattr(info, name) for name, _ in info._fields_}

    def run(self):
        st = self._lib.moe_rerouting_v2(self._pargs, self._ws, self._wsb, self._s)
        if st != _lib.SUCCESS:
            _raise(st, "moe_rerouting_v2")

    def run_noalloc(self):
        """The same call through moe_rerouting_v2_noalloc: the library's own
        scratch instead of this call's workspace (no allocation)."""
        st = self._lib.moe_rerouting_v2_noalloc(self._pargs, self._s)
        if st != _lib.SUCCESS:
            _raise(st, "moe_rerouting_v2_noalloc")

    def run_offsets(self):
        st = self._lib.moe_rerouting_v2_offsets(self._pargs, self._ws, self._wsb, self._s)
        if st != _lib.SUCCESS:
            _raise(st, "moe_rerouting_v2_offsets")

    def run_gather(self):
        st = self._lib.moe_rerouting_v2_gather(self._pargs, self._ws, self._wsb, self._s)
        if st != _lib.SUCCESS:
            _raise(st, "moe_rerouting_v2_gather")

    def device_status(self) -> int:
        return self._lib.mrr_get_device_status(self._ws, self._s)


def get_device_status(workspace: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> int:
    """Synchronizes the stream and returns the status code the last offsets
    phase left in `workspace` (0 = counts valid, 6 = bad counts)."""
    s = stream if stream is not None else torch.cuda.current_stream(workspace.device)
    return int(_lib.load().mrr_get_device_status(workspace.data_ptr(), s.cuda_stream))


def make_call(tokens, expert_token_num_per_rank, *, per_token_scales=None, expert_topk_weight=None,
              expert_token_num_type=1, idx_type=0, tokens_dtype=None, out=None, workspace=None,
              stream=None, direction=_lib.FORWARD):
    """Marshals once and returns (PreparedCall, outputs)."""
    args, outs = prepare(tokens, expert_token_num_per_rank, per_token_scales=per_token_scales,
                         expert_topk_weight=expert_topk_weight, expert_token_num_type=expert_token_num_type,
                         idx_type=idx_type, tokens_dtype=tokens_dtype, out=out, direction=direction)
    dev = tokens.device
    need = workspace_size(args.A, args.N, args.E)
    if need == 0:
        raise MrrValueError(_lib.ERROR_INVALID_SHAPE, "mrr_workspace_size")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, dev)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
        if s != torch.cuda.current_stream(dev):
            workspace.record_stream(s)
    keep = (tokens, expert_token_num_per_rank, per_token_scales, expert_topk_weight) + tuple(outs)
    return PreparedCall(args, workspace, s, keep), outs


def _run(direction, tokens, expert_token_num_per_rank, per_token_scales, expert_topk_weight,
         expert_token_num_type, idx_type, tokens_dtype, check, workspace, where):
    with torch.cuda.device(tokens.device):
        call, outs = make_call(tokens, expert_token_num_per_rank, per_token_scales=per_token_scales,
                               expert_topk_weight=expert_topk_weight,
                               expert_token_num_type=expert_token_num_type, idx_type=idx_type,
                               tokens_dtype=tokens_dtype, workspace=workspace, direction=direction)
        call.run()
        if check:
            st = call.device_status()
            if st != _lib.SUCCESS:
                _raise(st, where)
    return outs


def moe_re_routing(tokens: torch.Tensor, expert_token_num_per_rank: torch.Tensor, *,
                   per_token_scales: Optional[torch.Tensor] = None,
                   expert_topk_weight: Optional[torch.Tensor] = None,
                   expert_token_num_type: int = 1, idx_type: int = 0,
                   tokens_dtype: Optional[str] = None, check: bool = False,
                   workspace: Optional[torch.Tensor] = None):
    """Re-routes rank-major tokens into expert-major order on the GPU.

    Returns (permute_tokens, permute_per_token_scales, permute_token_idx,
    expert_token_num, permute_topk_weight). Asynchronous on the current stream.
    Count values are checked on the device; with check=True the call waits
    for the stream and raises MrrValueError when they were invalid (then the
    outputs were not written)."""
    return _run(_lib.FORWARD, tokens, expert_token_num_per_rank, per_token_scales, expert_topk_weight,
                expert_token_num_type, idx_type, tokens_dtype, check, workspace, "device count check")


def moe_re_routing_inverse(tokens: torch.Tensor, expert_token_num_per_rank: torch.Tensor, *,
                           per_token_scales: Optional[torch.Tensor] = None,
                           expert_topk_weight: Optional[torch.Tensor] = None,
                           expert_token_num_type: int = 1, idx_type: int = 0,
                           tokens_dtype: Optional[str] = None, check: bool = False,
                           workspace: Optional[torch.Tensor] = None):
    """The inverse re-route: `tokens` (and the optional scales and weights)
    are rows in expert-major order, as moe_re_routing returns them; they come
    back in rank-major order, row DstOffset(i,j) + k going to row
    SrcOffset(i,j) + k. Same arguments and result tuple as moe_re_routing;
    permute_token_idx is relative to this call's input and output (gather:
    output row s came from input row idx[s]), which makes it the forward
    call's scatter index and vice versa."""
    return _run(_lib.INVERSE, tokens, expert_token_num_per_rank, per_token_scales, expert_topk_weight,
                expert_token_num_type, idx_type, tokens_dtype, check, workspace, "device count check")
