"""Seeded synthetic inputs for the MoE re-routing operator.

This module only draws inputs: it holds none of the operator's arithmetic (no
offsets, no moves). Both the CPU oracle and the HIP path are fed from it.

The five named workloads follow the shapes of the pages' examples:
  * "tiny": N=2, E=4, counts uniform in [1, 8], H=128 fp16 tokens, [A] fp32
    scales; the smallest case, used for the smoke check;
  * "pages_shape": the single-operator example of the torch_npu V1 page
    (npu_moe_re_routing, "调用示例") and of the MoeReRoutingV2 article
    ("PyTorch API 调用"): A=16384, H=7168 int8 tokens in [-10, 20), N=E=16.
    The V1 generator overrides every random draw with 1, so every count is 1
    except the last cell, which takes the remainder 16384 - 255;
  * "balanced_bf16": same A and H, bf16 tokens, counts 1 + a uniform
    multinomial over the 256 cells, int64 counts, top-k weights;
  * "mxfp8_skewed": N=32, E=8, A=32768 fp8-e4m3 tokens, Zipf(1.2) cell
    weights, e8m0 scales [A, H/64, 2], top-k weights, scatter index;
  * "tiny_segments": N=256, E=64, A=65536, fp4 tokens packed two per byte
    (H=2048, 1024 bytes a row), [A, 32] fp32 scales, top-k weights.
Two more stand for shapes the examples leave out: "odd_rows" (H=79 f16
rows, 158 bytes) and "experts_384" (a 384-cell count matrix, N=16 x E=24,
A=16384 fp8 rows of 7168 bytes). No public dataset is named by the pages;
these synthetic draws stand in for the all-to-all output the operator would
receive.

Token arrays hold raw bits: bf16 as uint16, fp8/hif8/fp4 as uint8, fp16 as
float16, int8 as int8. Casts from float32 go through torch on the CPU
(round-to-nearest-even), so every consumer sees identical bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# token dtype name -> (bits per element, numpy storage dtype)
TOKEN_DTYPES = {
    "float16": (16, np.float16),
    "bfloat16": (16, np.uint16),
    "int8": (8, np.int8),
    "float8_e5m2": (8, np.uint8),
    "float8_e4m3fn": (8, np.uint8),
    "hifloat8": (8, np.uint8),
    "float4_e2m1fn_x2": (4, np.uint8),
    "float4_e1m2fn_x2": (4, np.uint8),
}


@dataclass
class Workload:
    name: str
    counts: np.ndarray                 # [N, E] int32 | int64
    tokens: np.ndarray                 # [A, H*bits/8 / itemsize] raw bits
    tokens_dtype: str                  # key of TOKEN_DTYPES
    H: int                             # logical token length
    scales: Optional[np.ndarray] = None        # [A] | [A,S] float32, or [A, ceil(H/64), 2] uint8 (e8m0)
    scales_dtype: Optional[str] = None         # "float32" | "float8_e8m0fnu"
    weight: Optional[np.ndarray] = None        # [A, 1] float32
    etn_type: int = 1
    idx_type: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def A(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def N(self) -> int:
        return int(self.counts.shape[0])

    @property
    def E(self) -> int:
        return int(self.counts.shape[1])

    @property
    def token_row_bytes(self) -> int:
        return self.H * TOKEN_DTYPES[self.tokens_dtype][0] // 8

    @property
    def scale_row_bytes(self) -> int:
        if self.scales is None or self.A == 0:
            return 0
        return self.scales.nbytes // self.A

    def algorithmic_bytes(self) -> int:
        """Bytes the operator must move: token and scale rows and weights read and
        written, the index written, the counts read and expert_token_num written."""
        a = self.A
        cb = self.counts.dtype.itemsize
        total = 2 * a * self.token_row_bytes + 4 * a
        total += 2 * a * self.scale_row_bytes
        if self.weight is not None:
            total += 8 * a
        total += self.N * self.E * cb + self.E * cb
        return total


def _f32_to_bits(x: np.ndarray, torch_dtype_name: str) -> np.ndarray:
    import torch  # CPU-only use: round-to-nearest-even casts

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    tdt = getattr(torch, torch_dtype_name)
    y = t.to(tdt)
    if y.element_size() == 2:
        return y.view(torch.uint16).numpy().copy()
    return y.view(torch.uint8).numpy().copy()


def tiny(seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, 9, (2, 4), dtype=np.int32)
    a = int(counts.sum())
    tokens = rng.standard_normal((a, 128), dtype=np.float32).astype(np.float16)
    scales = rng.standard_normal(a, dtype=np.float32)
    return Workload("tiny", counts, tokens, "float16", 128, scales, "float32", None, 1, 0)


def pages_shape(seed: int = 2) -> Workload:
    rng = np.random.default_rng(seed)
    n = e = 16
    a, h = 16384, 7168
    counts = np.ones((n, e), np.int32)
    counts[n - 1, e - 1] = a - (n * e - 1)
    tokens = rng.integers(-10, 20, (a, h), dtype=np.int8)
    scales = rng.standard_normal(a, dtype=np.float32)
    return Workload("pages_shape", counts, tokens, "int8", h, scales, "float32", None, 1, 0)


def balanced_bf16(seed: int = 3) -> Workload:
    rng = np.random.default_rng(seed)
    n = e = 16
    a, h = 16384, 7168
    counts = (1 + rng.multinomial(a - n * e, [1.0 / (n * e)] * (n * e))).reshape(n, e).astype(np.int64)
    tokens = _f32_to_bits(rng.standard_normal((a, h), dtype=np.float32), "bfloat16")
    weight = rng.random((a, 1), dtype=np.float32)
    return Workload("balanced_bf16", counts, tokens, "bfloat16", h, None, None, weight, 1, 0)


def mxfp8_skewed(seed: int = 4) -> Workload:
    rng = np.random.default_rng(seed)
    n, e = 32, 8
    a, h = 32768, 7168
    p = (np.arange(n * e) + 1.0) ** -1.2
    p /= p.sum()
    counts = (1 + rng.multinomial(a - n * e, p)).reshape(n, e).astype(np.int32)
    f = np.clip(rng.standard_normal((a, h), dtype=np.float32), -448.0, 448.0)
    tokens = _f32_to_bits(f, "float8_e4m3fn")
    scales = rng.integers(120, 135, (a, h // 64, 2), dtype=np.uint8)
    weight = rng.random((a, 1), dtype=np.float32)
    return Workload("mxfp8_skewed", counts, tokens, "float8_e4m3fn", h, scales, "float8_e8m0fnu",
                    weight, 1, 1)


def tiny_segments(seed: int = 5) -> Workload:
    rng = np.random.default_rng(seed)
    n, e = 256, 64
    a, h = 65536, 2048
    counts = (1 + rng.multinomial(a - n * e, [1.0 / (n * e)] * (n * e))).reshape(n, e).astype(np.int32)
    tokens = rng.integers(0, 256, (a, h // 2), dtype=np.uint8)
    scales = rng.standard_normal((a, 32), dtype=np.float32)
    weight = rng.random((a, 1), dtype=np.float32)
    return Workload("tiny_segments", counts, tokens, "float4_e2m1fn_x2", h, scales, "float32",
                    weight, 1, 0)


def experts_384(seed: int = 7) -> Workload:
    """A count matrix of 384 cells, the size of a 384-expert model's expert
    set spread over 16 ranks (N=16, E=24 local experts): A=16384 fp8-e4m3
    tokens of H=7168, counts 1 + a uniform multinomial, [A] fp32 per-token
    scales, top-k weights."""
    rng = np.random.default_rng(seed)
    n, e = 16, 24
    a, h = 16384, 7168
    counts = (1 + rng.multinomial(a - n * e, [1.0 / (n * e)] * (n * e))).reshape(n, e).astype(np.int32)
    tokens = rng.integers(0, 256, (a, h), dtype=np.uint8)
    scales = rng.standard_normal(a, dtype=np.float32)
    weight = rng.random((a, 1), dtype=np.float32)
    return Workload("experts_384", counts, tokens, "float8_e4m3fn", h, scales, "float32", weight, 1, 0)


def odd_rows(seed: int = 6) -> Workload:
    """Rows that are no multiple of 4 bytes: H = 79 f16 (158 bytes, the odd H
    of the pages' graph-mode sample) over 262,144 tokens, balanced 16 x 16
    counts, [A] fp32 scales."""
    rng = np.random.default_rng(seed)
    n = e = 16
    a, h = 262144, 79
    counts = (1 + rng.multinomial(a - n * e, [1.0 / (n * e)] * (n * e))).reshape(n, e).astype(np.int32)
    tokens = rng.standard_normal((a, h), dtype=np.float32).astype(np.float16)
    scales = rng.standard_normal(a, dtype=np.float32)
    return Workload("odd_rows", counts, tokens, "float16", h, scales, "float32", None, 1, 0)


CONFIGS = {
    "tiny": tiny,
    "pages_shape": pages_shape,
    "balanced_bf16": balanced_bf16,
    "mxfp8_skewed": mxfp8_skewed,
    "tiny_segments": tiny_segments,
    "odd_rows": odd_rows,
    "experts_384": experts_384,
}


def make(name: str) -> Workload:
    return CONFIGS[name]()


def random_case(seed: int, N: int, E: int, H: int, *, tokens_dtype: str = "float16",
                counts_dtype=np.int32, count_range=(0, 6), scales: Optional[str] = None,
                S: int = 1, weight: bool = False, etn_type: int = 1, idx_type: int = 0) -> Workload:
    """A fuzz case. Token rows are uniform random bits (so NaN payloads, -0 and
    subnormals appear); counts are uniform in [lo, hi), so zero counts (empty
    segments) appear when lo == 0. scales: None | "a" ([A] f32) | "as" ([A,S]
    f32) | "e8m0" ([A, ceil(H/64), 2] bytes)."""
    rng = np.random.default_rng(seed)
    lo, hi = count_range
    counts = rng.integers(lo, hi, (N, E)).astype(counts_dtype)
    a = int(counts.sum())
    bits, np_dt = TOKEN_DTYPES[tokens_dtype]
    row_bytes = H * bits // 8
    raw = rng.integers(0, 256, (a, row_bytes), dtype=np.uint8)
    tokens = raw.view(np_dt).reshape(a, row_bytes // np.dtype(np_dt).itemsize)
    sc, sc_dt = None, None
    if scales == "a":
        sc, sc_dt = rng.integers(0, 256, (a, 4), dtype=np.uint8).view(np.float32).reshape(a), "float32"
    elif scales == "as":
        sc, sc_dt = rng.integers(0, 256, (a, 4 * S), dtype=np.uint8).view(np.float32).reshape(a, S), "float32"
    elif scales == "e8m0":
        sc, sc_dt = rng.integers(0, 256, (a, (H + 63) // 64, 2), dtype=np.uint8), "float8_e8m0fnu"
    elif scales is not None:
        raise ValueError(scales)
    w = rng.integers(0, 256, (a, 4), dtype=np.uint8).view(np.float32).reshape(a, 1) if weight else None
    return Workload(f"random_{seed}", counts, tokens, tokens_dtype, H, sc, sc_dt, w, etn_type, idx_type)


def torch_inputs(w: Workload, device="cuda"):
    """The workload as torch tensors on `device`, with the operator's dtypes."""
    import torch

    dev = torch.device(device)
    tok = torch.from_numpy(np.ascontiguousarray(w.tokens))
    tok_dtype = {
        "float16": torch.float16, "bfloat16": torch.bfloat16, "int8": torch.int8,
        "float8_e5m2": torch.float8_e5m2, "float8_e4m3fn": torch.float8_e4m3fn,
        "hifloat8": torch.uint8, "float4_e2m1fn_x2": torch.uint8, "float4_e1m2fn_x2": torch.uint8,
    }[w.tokens_dtype]
    tok = tok.view(tok_dtype).to(dev)
    out = {"tokens": tok, "counts": torch.from_numpy(w.counts.copy()).to(dev),
           "tokens_dtype": None if w.tokens_dtype not in ("hifloat8", "float4_e2m1fn_x2", "float4_e1m2fn_x2")
           else w.tokens_dtype}
    if w.scales is not None:
        s = torch.from_numpy(np.ascontiguousarray(w.scales))
        if w.scales_dtype == "float8_e8m0fnu":
            s = s.view(torch.float8_e8m0fnu)
        out["scales"] = s.to(dev)
    else:
        out["scales"] = None
    out["weight"] = None if w.weight is None else torch.from_numpy(w.weight.copy()).to(dev)
    return out
