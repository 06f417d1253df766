"""The C-ABI library on the host, without a GPU: it loads, exports every
function include/moe_rerouting_v2.h declares, and its host checks
(mrr_validate, the same checks every launching call makes first) accept the
operator's contract and reject everything outside it with the right code.

Pointers here are fake addresses: mrr_validate compares them and tests their
alignment but never dereferences them, and makes no HIP call."""
import ctypes
import os
import re

import pytest

from moe_token_re_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADER = os.path.join(INCLUDE, "moe_rerouting_v2.h")
# header -> the library that must export what it declares
LIBRARIES = {"moe_rerouting_v2.h": _lib.LIB_PATH,
             "mrr_bench_copy.h": os.path.join(os.path.dirname(_lib.LIB_PATH), "libmrr_bench_copy.so")}

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    headers = sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h"))
    assert headers == sorted(LIBRARIES), headers
    for h in headers:
        lib = ctypes.CDLL(LIBRARIES[h])
        for n in declared_functions(os.path.join(INCLUDE, h)):
            assert hasattr(lib, n), (h, n)


def test_status_strings():
    for code, name in [(0, "MRR_SUCCESS"), (1, "MRR_ERROR_INVALID_VALUE"), (2, "MRR_ERROR_INVALID_SHAPE"),
                       (3, "MRR_ERROR_UNSUPPORTED_DTYPE"), (4, "MRR_ERROR_MISALIGNED"),
                       (5, "MRR_ERROR_WORKSPACE_TOO_SMALL"), (6, "MRR_ERROR_BAD_COUNTS"), (7, "MRR_ERROR_HIP")]:
        assert _lib.status_string(code) == name


def test_workspace_size():
    L = _lib.load()
    # 256-byte header + round_up(8*(M+1), 256) for the pair table + round_up(4*A, 256) for the row map
    assert L.mrr_workspace_size(16384, 16, 16) == 256 + 1280 + 1024 + 65536
    assert L.mrr_workspace_size(65536, 256, 64) == 256 + 65792 + 65536 + 262144
    assert L.mrr_workspace_size(42, 2, 4) == 256 + 256 + 256
    assert L.mrr_workspace_size(0, 0, 5) == 256 + 256 + 0
    assert L.mrr_workspace_size(0, -1, 4) == 0
    assert L.mrr_workspace_size(-1, 2, 4) == 0
    assert L.mrr_workspace_size(1 << 31, 2, 4) == 0
    assert L.mrr_workspace_size(0, 1 << 20, 1 << 20) == 0


# Fake device addresses, far apart so that no two buffers overlap.
BASE = {"tokens": 0x1000000000, "counts": 0x2000000000, "scales": 0x3000000000, "weight": 0x4000000000,
        "p_tokens": 0x5000000000, "p_scales": 0x6000000000, "idx": 0x7000000000, "etn": 0x8000000000,
        "p_weight": 0x9000000000, "ws": 0xA000000000}


def valid_args(A=64, H=128, N=2, E=4, tok=_lib.F16, cnt=_lib.I32, scales="f32", weight=True):
    a = _lib.MrrArgs()
    a.tokens, a.tokens_dtype, a.A, a.H = BASE["tokens"], tok, A, H
    a.expert_token_num_per_rank, a.counts_dtype, a.N, a.E = BASE["counts"], cnt, N, E
    if scales == "f32":
        a.per_token_scales, a.scales_dtype, a.scales_ndim = BASE["scales"], _lib.F32, 1
        a.scales_dims[0] = A
    elif scales == "e8m0":
        a.per_token_scales, a.scales_dtype, a.scales_ndim = BASE["scales"], _lib.F8_E8M0, 3
        a.scales_dims[0], a.scales_dims[1], a.scales_dims[2] = A, (H + 63) // 64, 2
    if scales:
        a.permute_per_token_scales = BASE["p_scales"]
    if weight:
        a.expert_topk_weight, a.permute_topk_weight = BASE["weight"], BASE["p_weight"]
    a.permute_tokens, a.permute_token_idx, a.expert_token_num = BASE["p_tokens"], BASE["idx"], BASE["etn"]
    a.expert_token_num_type, a.idx_type = 1, 0
    return a


def validate(a, ws=BASE["ws"], ws_bytes=None):
    L = _lib.load()
    if ws_bytes is None:
        ws_bytes = L.mrr_workspace_size(min(max(a.A, 0), (1 << 31) - 1), max(a.N, 0), max(a.E, 0))
    return L.mrr_validate(ctypes.byref(a), ws, ws_bytes)


def test_valid_configurations():
    assert validate(valid_args()) == _lib.SUCCESS
    assert validate(valid_args(scales=None, weight=False)) == _lib.SUCCESS
    assert validate(valid_args(A=16384, H=7168, N=16, E=16, tok=_lib.I8)) == _lib.SUCCESS
    assert validate(valid_args(A=32768, H=7168, N=32, E=8, tok=_lib.F8_E4M3FN, scales="e8m0")) == _lib.SUCCESS
    assert validate(valid_args(A=65536, H=2048, N=256, E=64, tok=_lib.F4_E2M1)) == _lib.SUCCESS
    assert validate(valid_args(H=79, scales="e8m0")) == _lib.SUCCESS   # odd rows, 2 scale pairs
    assert validate(valid_args(H=16383, tok=_lib.I8)) == _lib.SUCCESS
    a = valid_args(A=0, N=3, E=2)
    assert validate(a) == _lib.SUCCESS                                 # empty input
    a = valid_args(A=0, N=0, E=3)
    assert validate(a) == _lib.SUCCESS
    a = valid_args(A=0, N=0, E=0)
    a.expert_token_num = None
    assert validate(a) == _lib.SUCCESS
    for t in range(_lib.F16, _lib.F4_E1M2 + 1):
        assert validate(valid_args(tok=t)) == _lib.SUCCESS
    a = valid_args()
    a.scales_ndim, a.scales_dims[1] = 2, 32
    assert validate(a) == _lib.SUCCESS
    a = valid_args(scales=None)
    a.permute_per_token_scales = None                                  # absent scales: output unused
    assert validate(a) == _lib.SUCCESS
    a = valid_args(scales=None)
    a.permute_per_token_scales = BASE["p_scales"]
    assert validate(a) == _lib.SUCCESS
    a = valid_args(tok=_lib.I8, H=33)
    a.tokens += 1                                                      # byte rows: any alignment
    a.permute_tokens += 3
    assert validate(a) == _lib.SUCCESS
    a = valid_args(scales="e8m0")
    a.direction = _lib.INVERSE                                         # the same checks run backwards
    assert validate(a) == _lib.SUCCESS


def _with(f, **kw):
    a = valid_args(**kw)
    f(a)
    return a


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "tokens_dtype", _lib.I32), _lib.ERROR_UNSUPPORTED_DTYPE),
    (lambda a: setattr(a, "tokens_dtype", 99), _lib.ERROR_UNSUPPORTED_DTYPE),
    (lambda a: setattr(a, "counts_dtype", _lib.F32), _lib.ERROR_UNSUPPORTED_DTYPE),
    (lambda a: setattr(a, "scales_dtype", _lib.F16), _lib.ERROR_UNSUPPORTED_DTYPE),
    (lambda a: setattr(a, "expert_token_num_type", 2), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "idx_type", -1), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "direction", 2), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "direction", -1), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "H", 0), _lib.ERROR_INVALID_SHAPE),
    (lambda a: setattr(a, "H", 16384), _lib.ERROR_INVALID_SHAPE),
    (lambda a: setattr(a, "A", -1), _lib.ERROR_INVALID_SHAPE),
    (lambda a: setattr(a, "A", 1 << 31), _lib.ERROR_INVALID_SHAPE),
    (lambda a: setattr(a, "N", -2), _lib.ERROR_INVALID_SHAPE),
    (lambda a: (setattr(a, "N", 0)), _lib.ERROR_INVALID_SHAPE),          # no cells but A > 0
    (lambda a: setattr(a, "scales_ndim", 4), _lib.ERROR_INVALID_SHAPE),
    (lambda a: a.scales_dims.__setitem__(0, 63), _lib.ERROR_INVALID_SHAPE),
    (lambda a: (setattr(a, "scales_ndim", 2), a.scales_dims.__setitem__(1, 0)), _lib.ERROR_INVALID_SHAPE),
    (lambda a: setattr(a, "permute_topk_weight", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "expert_topk_weight", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "permute_per_token_scales", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "tokens", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "permute_tokens", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "permute_token_idx", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "expert_token_num", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "expert_token_num_per_rank", None), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "permute_token_idx", BASE["idx"] + 2), _lib.ERROR_MISALIGNED),
    (lambda a: setattr(a, "expert_token_num_per_rank", BASE["counts"] + 2), _lib.ERROR_MISALIGNED),
    (lambda a: setattr(a, "expert_token_num", BASE["etn"] + 1), _lib.ERROR_MISALIGNED),
    (lambda a: setattr(a, "expert_topk_weight", BASE["weight"] + 2), _lib.ERROR_MISALIGNED),
    (lambda a: setattr(a, "permute_per_token_scales", BASE["p_scales"] + 1), _lib.ERROR_MISALIGNED),
    # overlaps: an output over an input, over another output, over the workspace
    (lambda a: setattr(a, "permute_tokens", BASE["tokens"] + 64), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "permute_token_idx", BASE["p_tokens"] + 1024), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "expert_token_num", BASE["ws"] + 16), _lib.ERROR_INVALID_VALUE),
    (lambda a: setattr(a, "permute_topk_weight", BASE["counts"]), _lib.ERROR_INVALID_VALUE),
])
def test_rejections(mutate, code):
    a = valid_args()
    mutate(a)
    assert validate(a) == code


def describe(a, ws=BASE["ws"]):
    L = _lib.load()
    info = _lib.MrrPlanInfo()
    st = L.mrr_describe_plan(ctypes.byref(a), ws, L.mrr_workspace_size(a.A, a.N, a.E), ctypes.byref(info))
    return st, info


def test_describe_plan():
    # pages' shape: 7168-byte rows in 16-byte vectors; 112 MiB of token rows take the one-launch
    # stream kernel: 64-lane workgroups, 16384 / 256 item waves, then one per KiB of the input rows
    st, info = describe(valid_args(A=16384, H=7168, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS
    assert info.fused == 2 and info.one_launch_workgroups == 16384 // 256 + 16384 * 7
    # the two phases: the offsets kernel, then the stream gather over 64-vector chunks of the
    # token rows (16384 * 448 / 64) and chunks of 256 rows' items (index, and the 4-byte scale
    # rows with them)
    assert info.gather_kernel == 1 and info.token_vec_bytes == 16
    assert info.token_row_bytes == 7168 and info.scale_row_bytes == 4 and info.scale_vec_bytes == 4
    assert info.threads_per_workgroup == 64 and info.gather_workgroups == 114688 + 16384 // 256
    assert info.offsets_workgroups == 64           # the row map: one workgroup per 256 rows (<= 256 cells)
    # a smaller call with the same counts: the same one-launch kernel, whatever the size
    st, info = describe(valid_args(A=2048, H=7168, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 2 and info.one_launch_workgroups == 2048 // 256 + 2048 * 7
    # rows of 16-byte vectors that are no whole number of KiB (7184 bytes): the same kernel, its 1 KiB
    # chunks of the input rows taken as one stream (a chunk may reach into the next row)
    st, info = describe(valid_args(A=2048, H=7184, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 2 and info.one_launch_workgroups == 2048 // 256 + 2048 * 449 // 64
    # rows under 1 KiB (1008 bytes): one kernel of 256-thread workgroups that each recompute the offsets of
    # the (small) count matrix
    st, info = describe(valid_args(A=2048, H=1008, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 1 and info.threads_per_workgroup == 256
    assert info.one_launch_workgroups == info.gather_workgroups
    assert info.scale_inline_bytes == 4            # one 4-byte piece per row, loaded with the tokens
    rows = max(1, info.threads_per_workgroup * 8 // 63)
    assert info.rows_per_workgroup == min(rows, 256)
    assert info.gather_workgroups == -(-2048 // info.rows_per_workgroup)
    # 256x64 counts are too many to recompute per workgroup: two kernels
    st, info = describe(valid_args(A=65536, H=2048, N=256, E=64, tok=_lib.F4_E2M1))
    assert st == _lib.SUCCESS and info.fused == 0 and info.token_row_bytes == 1024
    assert info.offsets_workgroups == 16 * 8       # bands of 1024 // 64 = 16 ranks, 8 workgroups each
    # the banded offsets kernel: more than 1024 cells, at most 1024 experts and 2^17 cells
    for n, e, wgs in [(1, 1024, 1), (2, 1024, 2), (33, 32, 2), (7, 513, 7), (5000, 1, 5), (512, 256, 128),
                      (2, 1025, 1), (520, 256, 1)]:
        st, info = describe(valid_args(A=0, N=n, E=e))
        assert st == _lib.SUCCESS and info.offsets_workgroups == wgs, (n, e)
    # e8m0 scales [A, 112, 2] of H=7168 fp8 tokens: 224-byte scale rows in 16-byte pieces
    st, info = describe(valid_args(A=32768, H=7168, N=32, E=8, tok=_lib.F8_E4M3FN, scales="e8m0"))
    assert st == _lib.SUCCESS and info.scale_row_bytes == 224 and info.scale_inline_bytes == 16
    # more scale pieces than threads: a separate scale pass
    a = valid_args(A=4096, H=64, tok=_lib.F16)
    a.scales_ndim, a.scales_dims[1] = 2, 5
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.rows_per_workgroup == 256 and info.scale_inline_bytes == 0
    # odd rows fall back to narrower vectors in the single-kernel path
    a = valid_args(tok=_lib.F16, H=79)
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.token_vec_bytes == 2 and info.token_row_bytes == 158
    # ...and take the one-launch kernel's byte form from 2 MiB of rows: 1024 item waves, then one
    # wave per KiB of the 158-byte rows taken as one stream.
    # In two phases they stream as aligned 16-byte blocks of the output in the stream gather: 1 KiB
    # chunks of the rows, and 256-row chunks of the items with their 4-byte scale rows
    st, info = describe(valid_args(tok=_lib.F16, H=79, A=262144, N=16, E=16))
    assert st == _lib.SUCCESS and info.fused == 2 and info.token_vec_bytes == 16
    assert info.one_launch_workgroups == 262144 // 256 + (262144 * 158 + 1023) // 1024
    assert info.gather_kernel == 1
    assert info.gather_workgroups == (262144 * 158 + 1023) // 1024 + 262144 // 256
    # rows under 147 bytes: the same (in two phases the same 1 KiB chunks, their row-map words
    # loaded one per lane)
    st, info = describe(valid_args(tok=_lib.F16, H=63, A=65536, N=16, E=16))
    assert st == _lib.SUCCESS and info.gather_kernel == 1 and info.fused == 2
    assert info.one_launch_workgroups == 65536 // 256 + (65536 * 126 + 1023) // 1024
    assert info.gather_workgroups == (65536 * 126 + 1023) // 1024 + 65536 // 256
    # the byte form wants both token buffers 16-byte aligned and fewer than 2^31 token bytes
    a = valid_args(tok=_lib.F16, H=79, A=262144, N=16, E=16)
    a.tokens = BASE["tokens"] + 2
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.fused != 2
    st, info = describe(valid_args(tok=_lib.I8, H=8191, A=262144, N=16, E=16))
    assert st == _lib.SUCCESS and info.fused == 2
    st, info = describe(valid_args(tok=_lib.I8, H=8193, A=262144, N=16, E=16))
    assert st == _lib.SUCCESS and info.fused == 0
    # scale rows of more than 16 bytes keep chunks of their own (e8m0 [A, 112, 2]: 224 bytes a row)
    st, info = describe(valid_args(A=32768, H=7168, N=32, E=8, tok=_lib.F8_E4M3FN, scales="e8m0"))
    assert st == _lib.SUCCESS and info.gather_kernel == 1
    assert info.gather_workgroups == 32768 * 448 // 64 + 32768 * 14 // 64 + 32768 // 256
    # empty input: nothing to gather, never the single-kernel path
    st, info = describe(valid_args(A=0, N=3, E=2))
    assert st == _lib.SUCCESS and info.fused == 0 and info.gather_workgroups == 0
    assert info.one_launch_workgroups == 0
    assert info.offsets_workgroups == 1
    st, info = describe(valid_args(A=0, N=0, E=2))
    assert st == _lib.SUCCESS and info.offsets_workgroups == 0
    # describe runs the same checks
    a = valid_args()
    a.idx_type = 3
    assert describe(a)[0] == _lib.ERROR_INVALID_VALUE
    assert _lib.load().mrr_describe_plan(ctypes.byref(valid_args()), BASE["ws"], 1 << 20, None) == \
        _lib.ERROR_INVALID_VALUE


def test_plan_size_classes():
    """The launch choices by count-matrix size and token bytes (launch shape
    only; every choice computes the same bytes)."""
    mib = 1 << 20
    # token rows of whole KiB (7168 bytes), at most 256 cells: the one-launch stream kernel at any size
    for n, e in [(8, 8), (4, 4), (1, 64), (16, 16)]:
        for a_rows in (1, 100, 48 * mib // 7168 + 1):
            st, info = describe(valid_args(A=a_rows, H=7168, N=n, E=e, tok=_lib.I8))
            assert st == _lib.SUCCESS and info.fused == 2, (n, e, a_rows)
            assert info.one_launch_workgroups == -(-a_rows // 256) + a_rows * 7
    # the same for rows of 16-byte vectors that are no whole number of KiB (7184 bytes: 449 vectors)
    for a_rows in (1, 100, 48 * mib // 7184 + 1):
        st, info = describe(valid_args(A=a_rows, H=7184, N=16, E=16, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 2, a_rows
        assert info.one_launch_workgroups == -(-a_rows // 256) + -(-a_rows * 449 // 64)
    # rows of 16-byte vectors under 1 KiB (1008 bytes): the fused kernel below 2 MiB of token rows where
    # it applies (at most 256 cells), the one-launch kernel from there on, at any size
    below2, at2 = 2 * mib // 1008 - 1, 2 * mib // 1008 + 1
    for n, e in [(8, 8), (4, 4), (1, 64), (16, 16)]:
        st, info = describe(valid_args(A=below2, H=1008, N=n, E=e, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 1, (n, e)
        for a_rows in (at2, 100 * mib // 1008):
            st, info = describe(valid_args(A=a_rows, H=1008, N=n, E=e, tok=_lib.I8))
            assert st == _lib.SUCCESS and info.fused == 2, (n, e, a_rows)
            assert info.one_launch_workgroups == -(-a_rows // 256) + -(-a_rows * 63 // 64)
    # 257..512 cells (no fused kernel there): the one-launch kernel at every size
    for a_rows in (1, below2, at2):
        st, info = describe(valid_args(A=a_rows, H=1008, N=16, E=24, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 2, a_rows
    # 32-byte rows (two vectors): the one-launch kernel from 2 MiB; 16-byte rows never
    st, info = describe(valid_args(A=3 * mib // 32, H=32, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 2 and info.one_launch_workgroups == -(-3 * mib // 32 // 256) + \
        -(-3 * mib // 32 * 2 // 64)
    st, info = describe(valid_args(A=3 * mib // 16, H=16, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 1
    # 16-byte rows (never the one-launch kernel): the fused kernel up to 28 MiB of token rows with at most
    # 64 cells, 48 MiB with at most 256, else offsets + gather
    below28, above28, above48 = 28 * mib // 16 - 1, 28 * mib // 16 + 1, 48 * mib // 16 + 1
    for n, e in [(8, 8), (4, 4), (1, 64)]:
        st, info = describe(valid_args(A=below28, H=16, N=n, E=e, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 1, (n, e)
        st, info = describe(valid_args(A=above28, H=16, N=n, E=e, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 0 and info.gather_kernel == 1, (n, e)
        assert info.one_launch_workgroups == 0 and info.offsets_workgroups == -(-above28 // 256)
    st, info = describe(valid_args(A=above28, H=16, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 1
    st, info = describe(valid_args(A=above48, H=16, N=16, E=16, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 0 and info.offsets_workgroups == -(-above48 // 256)
    # rows that are no multiple of 16 bytes take the one-launch kernel's byte form (one wave per KiB):
    # from 512 bytes (1000 here) at any size, shorter ones (158 bytes) from 256 KiB of rows, the fused
    # kernel below that; with more than 512 cells offsets + gather
    for a_rows in (1, 42, 2 * mib // 1000 - 1, 2 * mib // 1000 + 1, 100 * mib // 1000):
        st, info = describe(valid_args(A=a_rows, H=1000, N=16, E=16, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 2, a_rows
        assert info.one_launch_workgroups == -(-a_rows // 256) + -(-a_rows * 1000 // 1024)
    for a_rows, fused in ((256 * 1024 // 158 - 1, 1), (256 * 1024 // 158 + 1, 2), (16 * mib // 158, 2)):
        st, info = describe(valid_args(A=a_rows, H=79, N=16, E=16, tok=_lib.F16))
        assert st == _lib.SUCCESS and info.fused == fused, a_rows
    for a_rows in (2 * mib // 1000 + 1, 100 * mib // 1000):
        st, info = describe(valid_args(A=a_rows, H=1000, N=16, E=40, tok=_lib.I8))
        assert st == _lib.SUCCESS and info.fused == 0 and info.gather_kernel == 1, a_rows
    # whole-KiB rows but not the one-launch kernel's other limits (above 48 MiB: offsets + gather)
    above48 = 48 * mib // 7168 + 1
    a = valid_args(A=above48, H=7168, N=16, E=16, tok=_lib.I8)
    a.scales_ndim, a.scales_dims[1] = 2, 1025                                      # 4100-byte scale rows
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.fused == 0
    a.scales_dims[1] = 1024                                                        # 4096 bytes: one launch
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.fused == 2
    # scale rows over 16 bytes: item waves of 64 output rows instead of 256
    assert info.one_launch_workgroups == -(-above48 // 64) + above48 * 7
    # 257..512 cells: the one-launch kernel too (eight cells a lane)
    for n, e in [(1, 257), (16, 32), (24, 16), (512, 1), (16, 24)]:
        for a_rows in (1, 3000, above48):
            st, info = describe(valid_args(A=a_rows, H=7168, N=n, E=e, tok=_lib.I8))
            assert st == _lib.SUCCESS and info.fused == 2, (n, e, a_rows)
            assert info.one_launch_workgroups == -(-a_rows // 256) + a_rows * 7
    st, info = describe(valid_args(A=above48, H=7168, N=1, E=513, tok=_lib.I8))   # 513 cells
    assert st == _lib.SUCCESS and info.fused == 0
    # 257..512 cells outside the one-launch kernel's limits (4100-byte scale rows): offsets + gather,
    # the offsets in 512-thread workgroups of 512 rows
    a = valid_args(A=3000, H=7168, N=16, E=32, tok=_lib.I8)
    a.scales_ndim, a.scales_dims[1] = 2, 1025
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.fused == 0 and info.offsets_workgroups == -(-3000 // 512)
    # 513..1024 cells: 1024-thread workgroups of 1024 rows
    st, info = describe(valid_args(A=3000, H=7168, N=32, E=32, tok=_lib.I8))
    assert st == _lib.SUCCESS and info.fused == 0 and info.offsets_workgroups == -(-3000 // 1024)


def test_int64_counts_alignment():
    a = valid_args(cnt=_lib.I64)
    assert validate(a) == _lib.SUCCESS
    a.expert_token_num_per_rank = BASE["counts"] + 4
    assert validate(a) == _lib.ERROR_MISALIGNED


def test_fp4_needs_even_h():
    assert validate(valid_args(tok=_lib.F4_E2M1, H=77)) == _lib.ERROR_INVALID_SHAPE
    assert validate(valid_args(tok=_lib.F4_E1M2, H=78)) == _lib.SUCCESS


def test_e8m0_shape_follows_h():
    a = valid_args(H=128, scales="e8m0")
    a.scales_dims[1] = 3
    assert validate(a) == _lib.ERROR_INVALID_SHAPE
    a = valid_args(H=128, scales="e8m0")
    a.scales_dims[2] = 1
    assert validate(a) == _lib.ERROR_INVALID_SHAPE


def test_workspace_checks():
    a = valid_args()
    need = _lib.load().mrr_workspace_size(64, 2, 4)
    assert validate(a, ws_bytes=need - 1) == _lib.ERROR_WORKSPACE_TOO_SMALL
    assert validate(a, ws=None) == _lib.ERROR_INVALID_VALUE
    assert validate(a, ws=BASE["ws"] + 8) == _lib.ERROR_MISALIGNED
    assert validate(a, ws=BASE["tokens"] + 128) == _lib.ERROR_INVALID_VALUE   # overlaps tokens


def test_launch_entry_points_reject_before_launch():
    """The launching calls run the same checks first: with bad arguments they
    return the error without touching the GPU (none is present here)."""
    L = _lib.load()
    a = valid_args()
    a.idx_type = 5
    ws = BASE["ws"]
    nb = L.mrr_workspace_size(64, 2, 4)
    for fn in (L.moe_rerouting_v2, L.moe_rerouting_v2_offsets, L.moe_rerouting_v2_gather):
        assert fn(ctypes.byref(a), ws, nb, None) == _lib.ERROR_INVALID_VALUE
    assert L.mrr_get_device_status(None, None) == _lib.ERROR_INVALID_VALUE


def test_gather_launches_stay_within_the_launch_limit():
    """A launch holds at most 2^32 - 1 threads: gathers with more workgroups
    than that are planned as several launches (the stream gather's 64-lane
    workgroups: at most 2^26 - 1 per launch; the row workgroups of 256 threads:
    at most 2^24 - 1)."""
    max64, max256 = ((1 << 32) - 1) // 64, ((1 << 32) - 1) // 256
    # 7168-byte int8 rows at odd addresses move one byte per lane: 112 token chunks per row,
    # plus A / 256 item chunks (which also move the 4-byte scale rows)
    for A, launches in [(599_000, 1), (600_000, 2)]:
        a = valid_args(A=A, H=7168, N=16, E=16, tok=_lib.I8, weight=False)
        a.tokens, a.permute_tokens = BASE["tokens"] + 1, BASE["p_tokens"] + 1
        st, info = describe(a)
        assert st == _lib.SUCCESS and info.gather_kernel == 1 and info.token_vec_bytes == 1
        chunks = A * 7168 // 64 + (-(-A // 256))
        assert info.gather_workgroups == chunks
        assert info.gather_launches == launches == -(-chunks // max64)
    # more than 2^31 stream chunks: the row-workgroup gather, one row per workgroup, in pieces
    far = 1 << 44  # 16 TiB apart: each buffer below fits between its neighbours
    A = (1 << 31) - 1
    a = valid_args(A=A, H=7168, N=16, E=16, tok=_lib.I8, weight=False)
    a.tokens, a.permute_tokens = far + 1, 2 * far + 1
    a.per_token_scales, a.permute_per_token_scales = 3 * far, 4 * far
    a.permute_token_idx, a.expert_token_num_per_rank, a.expert_token_num = 5 * far, 6 * far, 6 * far + 4096
    ws = 7 * far
    st, info = describe(a, ws=ws)
    assert st == _lib.SUCCESS and info.fused == 0 and info.gather_kernel == 0 and info.rows_per_workgroup == 1
    assert info.gather_workgroups == A and info.gather_launches == -(-A // max256)
    # A = 0: nothing to launch
    st, info = describe(valid_args(A=0, N=3, E=2))
    assert st == _lib.SUCCESS and info.gather_launches == 0
    st, info = describe(valid_args())
    assert st == _lib.SUCCESS and info.gather_launches == 1


def test_largest_count_matrix():
    """N * E up to 2^30 cells is accepted (the table's end entry then sits at
    int32 pair 2^30, word 2^31); one more is refused."""
    L = _lib.load()
    n = 1 << 15
    assert L.mrr_workspace_size(0, n, n) == 256 + 8 * ((1 << 30) + 1) + 248
    assert L.mrr_workspace_size(0, n + 1, n) == 0
    a = valid_args(A=0, N=n, E=n, scales=None, weight=False)
    st, info = describe(a)
    assert st == _lib.SUCCESS and info.offsets_workgroups == 1 and info.gather_kernel == 0
    a = valid_args(A=0, N=n + 1, E=n, scales=None, weight=False)
    assert validate(a, ws_bytes=1 << 40) == _lib.ERROR_INVALID_SHAPE


def test_noalloc_rejects_before_any_hip_call():
    """moe_rerouting_v2_noalloc refuses a call whose workspace would exceed the
    static scratch, and NULL arguments, before it touches the GPU (none is
    present here); its other checks are moe_rerouting_v2's."""
    L = _lib.load()
    assert L.moe_rerouting_v2_noalloc(None, None) == _lib.ERROR_INVALID_VALUE
    # 16 x 16 counts: the row map of A rows takes 4 A bytes of the 8 MiB scratch
    a_max = (_lib.NOALLOC_SCRATCH_BYTES - 256 - 2304) // 4
    assert L.mrr_workspace_size(a_max, 16, 16) <= _lib.NOALLOC_SCRATCH_BYTES
    assert L.mrr_workspace_size(a_max + 64, 16, 16) > _lib.NOALLOC_SCRATCH_BYTES
    a = valid_args(A=a_max + 64, H=64, N=16, E=16)
    assert L.moe_rerouting_v2_noalloc(ctypes.byref(a), None) == _lib.ERROR_WORKSPACE_TOO_SMALL
