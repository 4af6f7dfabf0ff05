"""Seeded synthetic inputs for the quantized linear GEMM.

This module is shared by the tests, the benchmark and the smoke check.  It
holds input preparation only -- random draws, rounding of the draws to
bfloat16, and the quantizers that turn them into 8-bit codes plus fp32
scales -- and none of the GEMM's arithmetic (no dot products, no scale
application, no output rounding).  Both the CPU oracle and the HIP library
consume the bytes it produces.

Formats and scale granularity follow "Building a High-Performance and
Portable vLLM Linear Backend with Helion", section "Helion Linear Backend /
Scope": FP8_Dynamic and W8A8_INT8 scale per activation token and per weight
output channel; Block_FP8 scales activations per 1x128 K group and weights
per 128x128 block.  The pages give no quantizer, so the scales are the
common dynamic choice: amax/448 for e4m3 (448 is the largest e4m3 value) and
amax/127 for symmetric int8; codes are round-to-nearest-even of x/scale,
clamped into range; an all-zero row/group/block gets scale 1.

Value distributions and shapes are those of the decoder linear layers the
pages evaluate (Qwen3 1.7B / 8B / 32B class): activations ~ N(0,1), some with
1% outlier channels scaled x20; weights ~ N(0, 0.02).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

try:  # torch supplies the float32 -> e4m3 / bf16 casts (round to nearest even)
    import torch
except Exception:  # pragma: no cover - torch is part of the image
    torch = None

E4M3_MAX = 448.0
INT8_MAX = 127.0

FORMATS = ("fp8", "int8", "block_fp8")


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, returned as float32."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn codes (uint8), nearest-even, saturated at +-448."""
    t = torch.from_numpy(np.ascontiguousarray(np.clip(x, -E4M3_MAX, E4M3_MAX), np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _safe_scale(amax: np.ndarray, qmax: float) -> np.ndarray:
    s = (amax.astype(np.float32) / np.float32(qmax)).astype(np.float32)
    s[amax == 0] = np.float32(1.0)
    return s


def quant_rows(x: np.ndarray, fmt: str):
    """Per-row (token or output channel) quantization. Returns (codes u8, scales f32)."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    if fmt == "int8":
        s = _safe_scale(amax, INT8_MAX)
        q = np.clip(np.rint(x / s[:, None]), -INT8_MAX, INT8_MAX).astype(np.int8)
        return q.view(np.uint8), s
    s = _safe_scale(amax, E4M3_MAX)
    return _e4m3_codes(x / s[:, None]), s


def quant_groups(x: np.ndarray, group: int = 128):
    """1 x group quantization of an activation [M,K] to e4m3: scales [M, K/group]."""
    x = np.asarray(x, np.float32)
    M, K = x.shape
    assert K % group == 0
    xg = x.reshape(M, K // group, group)
    s = _safe_scale(np.abs(xg).max(axis=2), E4M3_MAX)
    q = _e4m3_codes((xg / s[:, :, None]).reshape(M, K))
    return q, s


def quant_blocks(w: np.ndarray, block: int = 128):
    """block x block quantization of a weight [N,K] to e4m3: scales [N/block, K/block]."""
    w = np.asarray(w, np.float32)
    N, K = w.shape
    assert N % block == 0 and K % block == 0
    wb = w.reshape(N // block, block, K // block, block)
    s = _safe_scale(np.abs(wb).max(axis=(1, 3)), E4M3_MAX)
    q = _e4m3_codes((wb / s[:, None, :, None]).reshape(N, K))
    return q, s


def activations(M: int, K: int, key, outliers: bool = False, outlier_key=None) -> np.ndarray:
    """bf16-valued activations ~ N(0,1); optionally 1% outlier channels x20."""
    x = key.standard_normal((M, K), dtype=np.float32) if isinstance(key, np.random.Generator) \
        else rng(*key).standard_normal((M, K), dtype=np.float32)
    if outliers and K:
        g = outlier_key if isinstance(outlier_key, np.random.Generator) else rng(*outlier_key)
        cols = g.choice(K, size=max(1, int(round(0.01 * K))), replace=False)
        x[:, cols] *= np.float32(20.0)
    return bf16_round(x)


def norm_weight(K: int, key) -> np.ndarray:
    """bf16-valued RMS-norm weight [K] ~ 1 + N(0, 0.1) (a trained norm's gains
    sit near 1)."""
    return bf16_round((1.0 + 0.1 * rng(*key).standard_normal(K)).astype(np.float32))


def weights(N: int, K: int, key) -> np.ndarray:
    """bf16-valued weights ~ N(0, 0.02)."""
    g = key if isinstance(key, np.random.Generator) else rng(*key)
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return bf16_round(w)


@dataclass
class Case:
    """One GEMM problem: codes A [M,K], B [N,K] (uint8 views), fp32 scales."""
    fmt: str          # "fp8" | "int8" | "block_fp8"
    M: int
    N: int
    K: int
    A: np.ndarray
    sA: np.ndarray
    B: np.ndarray
    sB: np.ndarray
    tag: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def block(self) -> bool:
        return self.fmt == "block_fp8"


def quantize(fmt: str, x: np.ndarray, w: np.ndarray):
    if fmt == "block_fp8":
        A, sA = quant_groups(x)
        B, sB = quant_blocks(w)
    else:
        A, sA = quant_rows(x, fmt)
        B, sB = quant_rows(w, fmt)
    return A, sA, B, sB


@lru_cache(maxsize=4)
def quantized_weight(fmt: str, N: int, K: int, root: int = 0):
    """Codes and scales of the seeded weight [N,K] (shared by every M)."""
    w = weights(N, K, (root, 1, K, N))
    if fmt == "block_fp8":
        B, sB = quant_blocks(w)
    else:
        B, sB = quant_rows(w, fmt)
    return B, sB


def quantized_activation(fmt: str, M: int, K: int, root: int = 0, outliers: bool = False):
    x = activations(M, K, (root, 2, M, K), outliers=outliers, outlier_key=(root, 3, K))
    if fmt == "block_fp8":
        return quant_groups(x)
    return quant_rows(x, fmt)


def make_case(fmt: str, M: int, N: int, K: int, *, outliers: bool | None = None,
              root: int = 0, tag: str = "") -> Case:
    """The seeded recipe: B from SeedSequence([root,1,K,N]) (shared across M),
    A from [root,2,M,K], outlier channels from [root,3,K].  Outliers default
    to on for the FP8 formats and off for INT8."""
    if fmt not in FORMATS:
        raise ValueError(fmt)
    if outliers is None:
        outliers = fmt != "int8"
    B, sB = quantized_weight(fmt, N, K, root)
    A, sA = quantized_activation(fmt, M, K, root, outliers)
    return Case(fmt, M, N, K, A, sA, B, sB, tag=tag or f"{fmt}-M{M}-N{N}-K{K}")


def make_case_seed0(fmt: str, M: int, N: int, K: int) -> Case:
    """The small FP8 case stated with plain seed 0: A drawn first, then B, from
    one generator; activations without outliers."""
    g = np.random.Generator(np.random.PCG64(0))
    x = bf16_round(g.standard_normal((M, K), dtype=np.float32))
    w = bf16_round(g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    A, sA, B, sB = quantize(fmt, x, w)
    return Case(fmt, M, N, K, A, sA, B, sB, tag=f"{fmt}-seed0-M{M}-N{N}-K{K}")


# ---------------------------------------------------------------------------
# The workloads: decoder linear shapes (K, N) per model class and token counts.
# The decode token grid {1,2,4,8,16,24,32} is the one the pages tune on.
# ---------------------------------------------------------------------------
DECODE_M = (1, 2, 4, 8, 16, 24, 32)
SHAPES_1P7B = ((2048, 4096), (2048, 2048), (2048, 12288), (6144, 2048))
SHAPES_8B = ((4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096))
SHAPES_32B = ((5120, 10240), (8192, 5120), (5120, 51200), (25600, 5120))


def workload(name: str):
    """List of (fmt, M, N, K) points of a named workload."""
    if name == "fp8_small":
        return [("fp8", 16, 512, 1024)]
    if name == "int8_1p7b_decode":
        return [("int8", M, N, K) for (K, N) in SHAPES_1P7B for M in DECODE_M]
    if name == "fp8_8b":
        return [("fp8", M, N, K) for (K, N) in SHAPES_8B for M in DECODE_M + (128, 512)]
    if name == "block_fp8_8b":
        return [("block_fp8", M, N, K) for (K, N) in SHAPES_8B for M in DECODE_M + (512,)]
    if name == "all_32b":
        return [(f, M, N, K) for f in FORMATS for (K, N) in SHAPES_32B
                for M in DECODE_M + (2048,)]
    if name == "all_32b_decode":
        return [p for p in workload("all_32b") if p[1] <= 32]
    if name == "prefill":
        return [p for w in ("fp8_8b", "block_fp8_8b", "all_32b") for p in workload(w) if p[1] >= 512]
    raise KeyError(name)


# Mixture-of-experts layers of a 30B-class model with 3B active parameters
# (hidden 2048, 128 experts, 8 per token, expert width 768): gate_up
# (K=2048, N=1536) and down (K=768, N=2048), as (name, K, N).  Routing: each
# token picks 8 distinct experts uniformly (seeded); tokens sorted by expert.
MOE_LAYERS = (("gate_up", 2048, 1536), ("down", 768, 2048))
MOE_EXPERTS, MOE_TOPK = 128, 8


def moe_counts(batch: int, K: int, experts: int = MOE_EXPERTS, topk: int = MOE_TOPK) -> np.ndarray:
    """Rows per expert for a batch of tokens under seeded uniform top-k routing."""
    g = rng(83, batch, K)
    picks = np.stack([g.choice(experts, topk, replace=False) for _ in range(batch)])
    return np.bincount(picks.ravel(), minlength=experts)


def e4m3_codes(shape, key) -> np.ndarray:
    """Random finite e4m3 codes of both signs (timing inputs: no NaN codes)."""
    g = rng(*key)
    return (g.integers(0, 0x7E, shape, dtype=np.uint8) |
            (g.integers(0, 2, shape, dtype=np.uint8) << 7)).astype(np.uint8)


WORKLOADS = ("fp8_small", "int8_1p7b_decode", "fp8_8b", "block_fp8_8b", "all_32b", "all_32b_decode",
             "prefill")
