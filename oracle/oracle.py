"""ctypes binding of the CPU oracle (oracle.c) for MoeReRoutingV2.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg. The product path never imports this module, and
this module imports nothing from the product package.

The oracle treats every row as an opaque byte string, so callers pass numpy
arrays whose first axis is the token axis A; a row's byte size is the array's
bytes divided by A (fp4 tokens packed two per byte arrive as uint8 [A, H/2]).
The semantics are those of the page "CANN ops-transformer MoeReRoutingV2"
(nlpx.cn article), sections "计算公式" and "参数说明"; the readings taken where
that text is garbled are listed at the top of oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

OK = 0
BAD_ARGS = 1
BAD_COUNTS = 2


class OracleError(ValueError):
    """The oracle rejected its inputs (code BAD_ARGS or BAD_COUNTS)."""

    def __init__(self, code: int):
        super().__init__(f"oracle rejected the inputs (code {code})")
        self.code = code


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile oracle.c with gcc into a shared library (single-threaded, -O2)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
           "-I", _HERE, "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


def _counts_kind(counts: np.ndarray) -> int:
    if counts.dtype == np.int32:
        return 0
    if counts.dtype == np.int64:
        return 1
    raise TypeError(f"counts must be int32 or int64, got {counts.dtype}")


def allocate_outputs(tokens, counts, scales=None, weight=None):
    """Output arrays with the shapes and dtypes of the operator's results."""
    a = tokens.shape[0]
    return (np.empty_like(tokens),
            None if scales is None else np.empty_like(scales),
            np.empty((a,), np.int32),
            np.empty((counts.shape[1],), counts.dtype),
            None if weight is None else np.empty_like(weight))


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_offsets.argtypes = [vp, i32, i64, i64, vp, vp]
        lib.oracle_offsets.restype = i32
        lib.oracle_reroute.argtypes = [vp, i64, i64, vp, i32, i64, i64, vp, i64, vp,
                                       i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_reroute.restype = i32
        lib.oracle_reroute_inverse.argtypes = lib.oracle_reroute.argtypes
        lib.oracle_reroute_inverse.restype = i32
        self.lib = lib
        self.path = lib_path

    def offsets(self, counts: np.ndarray):
        """SrcOffset and DstOffset of every cell of counts[N, E], as int64 [N, E] arrays."""
        counts = np.ascontiguousarray(counts)
        if counts.ndim != 2:
            raise ValueError("counts must be 2-D [N, E]")
        n, e = counts.shape
        src = np.zeros((n, e), np.int64)
        dst = np.zeros((n, e), np.int64)
        rc = self.lib.oracle_offsets(_ptr(counts), _counts_kind(counts), n, e, _ptr(src), _ptr(dst))
        if rc != OK:
            raise OracleError(rc)
        return src, dst

    def reroute(self, tokens, counts, scales=None, weight=None, etn_type=1, idx_type=0, out=None):
        """Run the operator. Returns (permute_tokens, permute_scales or None,
        permute_token_idx int32 [A], expert_token_num [E] in the counts' dtype,
        permute_weight or None). `out` may hold preallocated arrays from
        allocate_outputs(), which are then filled and returned."""
        return self._call(self.lib.oracle_reroute, tokens, counts, scales, weight, etn_type, idx_type, out)

    def reroute_inverse(self, rows, counts, scales=None, weight=None, etn_type=1, idx_type=0, out=None):
        """The inverse re-route: expert-major rows (the operator's output
        layout) back to rank-major order. Same arguments and results as
        reroute()."""
        return self._call(self.lib.oracle_reroute_inverse, rows, counts, scales, weight, etn_type, idx_type, out)

    @staticmethod
    def _call(fn, tokens, counts, scales, weight, etn_type, idx_type, out):
        tokens = np.ascontiguousarray(tokens)
        counts = np.ascontiguousarray(counts)
        if counts.ndim != 2:
            raise ValueError("counts must be 2-D [N, E]")
        a = tokens.shape[0]
        row = tokens.nbytes // a if a else 0
        srow = 0
        if scales is not None:
            scales = np.ascontiguousarray(scales)
            if scales.shape[0] != a:
                raise ValueError("scales must have A rows")
            srow = scales.nbytes // a if a else 0
        if weight is not None:
            weight = np.ascontiguousarray(weight)
            if weight.dtype != np.float32 or weight.size != a:
                raise ValueError("weight must be float32 with A elements")
        outs = allocate_outputs(tokens, counts, scales, weight) if out is None else out
        o_tok, o_sc, o_idx, o_etn, o_w = outs
        rc = fn(_ptr(tokens), a, row, _ptr(counts), _counts_kind(counts), counts.shape[0],
                counts.shape[1], _ptr(scales), srow, _ptr(weight), int(etn_type), int(idx_type),
                _ptr(o_tok), _ptr(o_sc), _ptr(o_idx), _ptr(o_etn), _ptr(o_w))
        if rc != OK:
            raise OracleError(rc)
        return outs


def load() -> Oracle:
    """The oracle built from oracle.c, compiling it first when no build exists
    or the source is newer than the build."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB_PATH):
                build()
            _lib = Oracle(_LIB_PATH)
        return _lib


def offsets(counts):
    return load().offsets(counts)


def reroute(tokens, counts, scales=None, weight=None, etn_type=1, idx_type=0, out=None):
    return load().reroute(tokens, counts, scales, weight, etn_type, idx_type, out)


def reroute_inverse(rows, counts, scales=None, weight=None, etn_type=1, idx_type=0, out=None):
    return load().reroute_inverse(rows, counts, scales, weight, etn_type, idx_type, out)
