"""ctypes view of the C ABI in include/moe_rerouting_v2.h.

Loads the in-tree libmoe_rerouting_v2.so. There is no fallback: if the library
has not been built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_rerouting_v2.so")

# mrr_status
SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_INVALID_SHAPE = 2
ERROR_UNSUPPORTED_DTYPE = 3
ERROR_MISALIGNED = 4
ERROR_WORKSPACE_TOO_SMALL = 5
ERROR_BAD_COUNTS = 6
ERROR_HIP = 7

# mrr_args.direction
FORWARD = 0
INVERSE = 1

# mrr_dtype
F16, BF16, I8, F8_E5M2, F8_E4M3FN, HIF8, F4_E2M1, F4_E1M2, I32, I64, F32, F8_E8M0 = range(12)

EXPORTS = ("mrr_workspace_size", "mrr_validate", "mrr_describe_plan", "moe_rerouting_v2",
           "moe_rerouting_v2_offsets", "moe_rerouting_v2_gather", "mrr_get_device_status", "mrr_status_string",
           "mrr_source_hash", "moe_rerouting_v2_noalloc")
NOALLOC_SCRATCH_BYTES = 8 << 20  # MRR_NOALLOC_SCRATCH_BYTES


class MrrArgs(ctypes.Structure):
    """struct mrr_args, field for field."""

    _fields_ = [
        ("tokens", ctypes.c_void_p),
        ("tokens_dtype", ctypes.c_int32),
        ("A", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("expert_token_num_per_rank", ctypes.c_void_p),
        ("counts_dtype", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("E", ctypes.c_int64),
        ("per_token_scales", ctypes.c_void_p),
        ("scales_dtype", ctypes.c_int32),
        ("scales_ndim", ctypes.c_int32),
        ("scales_dims", ctypes.c_int64 * 3),
        ("expert_topk_weight", ctypes.c_void_p),
        ("permute_tokens", ctypes.c_void_p),
        ("permute_per_token_scales", ctypes.c_void_p),
        ("permute_token_idx", ctypes.c_void_p),
        ("expert_token_num", ctypes.c_void_p),
        ("permute_topk_weight", ctypes.c_void_p),
        ("expert_token_num_type", ctypes.c_int64),
        ("idx_type", ctypes.c_int64),
        ("direction", ctypes.c_int64),
    ]


class MrrPlanInfo(ctypes.Structure):
    """struct mrr_plan_info, field for field."""

    _fields_ = [
        ("fused", ctypes.c_int32),
        ("token_vec_bytes", ctypes.c_int32),
        ("scale_vec_bytes", ctypes.c_int32),
        ("rows_per_workgroup", ctypes.c_int32),
        ("threads_per_workgroup", ctypes.c_int32),
        ("gather_workgroups", ctypes.c_int64),
        ("token_row_bytes", ctypes.c_int64),
        ("scale_row_bytes", ctypes.c_int64),
        ("scale_inline_bytes", ctypes.c_int32),
        ("offsets_workgroups", ctypes.c_int64),
        ("gather_kernel", ctypes.c_int32),
        ("gather_launches", ctypes.c_int64),
        ("one_launch_workgroups", ctypes.c_int64),
    ]


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """The loaded library; raises RuntimeError if it has not been built, or was
    built from sources other than the ones beside it (mrr_source_hash)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m moe_token_re_amd.build` "
                    "(there is no CPU fallback)")
            from . import build

            lib = ctypes.CDLL(LIB_PATH)
            if not hasattr(lib, "mrr_source_hash"):
                raise RuntimeError(f"{LIB_PATH} carries no source hash: rebuild it "
                                   "with `python -m moe_token_re_amd.build`")
            lib.mrr_source_hash.argtypes = []
            lib.mrr_source_hash.restype = ctypes.c_char_p
            built, current = lib.mrr_source_hash().decode(), build.source_hash()
            if built != current:
                raise RuntimeError(f"{LIB_PATH} was built from other sources (hash {built}, sources {current}): "
                                   "rebuild it with `python -m moe_token_re_amd.build`")
            P = ctypes.POINTER(MrrArgs)
            vp, sz = ctypes.c_void_p, ctypes.c_size_t
            lib.mrr_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
            lib.mrr_workspace_size.restype = sz
            lib.mrr_validate.argtypes = [P, vp, sz]
            lib.mrr_validate.restype = ctypes.c_int
            lib.mrr_describe_plan.argtypes = [P, vp, sz, ctypes.POINTER(MrrPlanInfo)]
            lib.mrr_describe_plan.restype = ctypes.c_int
            for name in ("moe_rerouting_v2", "moe_rerouting_v2_offsets", "moe_rerouting_v2_gather"):
                fn = getattr(lib, name)
                fn.argtypes = [P, vp, sz, vp]
                fn.restype = ctypes.c_int
            lib.moe_rerouting_v2_noalloc.argtypes = [P, vp]
            lib.moe_rerouting_v2_noalloc.restype = ctypes.c_int
            lib.mrr_get_device_status.argtypes = [vp, vp]
            lib.mrr_get_device_status.restype = ctypes.c_int
            lib.mrr_status_string.argtypes = [ctypes.c_int]
            lib.mrr_status_string.restype = ctypes.c_char_p
            _lib = lib
        return _lib


def library_source_hash() -> str:
    """The source hash compiled into the loaded library (equal to the current
    sources' hash, or load() would have refused it)."""
    return load().mrr_source_hash().decode()


def status_string(code: int) -> str:
    return load().mrr_status_string(code).decode()
