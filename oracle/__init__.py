"""CPU oracle for the quantized linear GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``int8_gemm_linear_amd`` never imports it and shares no code with it.

The arithmetic lives in ``qlinear_oracle.c`` (plain C, double / int64
accumulation, bf16 round-to-nearest-even straight from double).  This module
only compiles it with gcc and marshals numpy arrays through ctypes.

Formats, restated from "Building a High-Performance and Portable vLLM Linear
Backend with Helion", section "Helion Linear Backend / Scope":
FP8_Dynamic and W8A8_INT8 carry one scale per activation token and one per
weight output channel; Block_FP8 carries one activation scale per 1x128 K
group and one weight scale per 128x128 weight block.

Every function here is pinned by ``tests/test_oracle.py`` against brute force
over exact rationals, torch's e4m3 and bf16 casts, numpy integer / float64
matrix products, closed forms and invariants.  No function is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_E4M3 = 0
FMT_INT8 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc -O2."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.orc_e4m3_to_double.restype = ctypes.c_double
    lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.orc_double_to_bf16.restype = ctypes.c_uint16
    lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_scaled_mm.restype = I
    lib.orc_scaled_mm.argtypes = [I, I, I64, I64, I64, P, I64, P, P, I64, P,
                                  P, I64, P, P, P, P, I]
    lib.orc_scaled_mm_points.restype = I
    lib.orc_scaled_mm_points.argtypes = [I, I, I64, I64, I64, P, I64, P, P, I64, P,
                                         I64, P, P, P, P, P, P, P, I]
    lib.orc_e4m3_decode_n.restype = None
    lib.orc_e4m3_decode_n.argtypes = [P, P, I64]
    lib.orc_double_to_bf16_n.restype = None
    lib.orc_double_to_bf16_n.argtypes = [P, P, I64]
    lib.orc_e4m3_nearest.restype = ctypes.c_uint8
    lib.orc_e4m3_nearest.argtypes = [ctypes.c_float]
    lib.orc_quant_per_token.restype = I
    lib.orc_quant_per_token.argtypes = [I, I64, I64, P, I64, P, I64, P]
    lib.orc_quant_per_group.restype = I
    lib.orc_quant_per_group.argtypes = [I64, I64, I64, P, I64, P, I64, P]
    lib.orc_rms_norm.restype = I
    lib.orc_rms_norm.argtypes = [I64, I64, P, I64, P, I64, P, ctypes.c_float, P, I64]
    lib.orc_silu_and_mul.restype = I
    lib.orc_silu_and_mul.argtypes = [I64, I64, P, I64, P, I64]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u8(x):
    x = np.asarray(x)
    if x.dtype != np.uint8:
        x = x.view(np.uint8)
    return np.ascontiguousarray(x)


def decode_e4m3(codes) -> np.ndarray:
    """OCP E4M3FN codes (uint8 array) -> float64 values."""
    c = _u8(codes)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_n(c.ctypes.data, out.ctypes.data, c.size)
    return out


def to_bf16_bits(x) -> np.ndarray:
    """float64 values -> bf16 bit patterns (uint16), nearest-even, one rounding."""
    d = np.ascontiguousarray(np.asarray(x, np.float64))
    out = np.empty(d.shape, np.uint16)
    _load().orc_double_to_bf16_n(d.ctypes.data, out.ctypes.data, d.size)
    return out


class Result:
    """Oracle outputs: ``y`` (bf16 bits [M,N]), ``ydbl`` (value before the
    final rounding), ``bound`` (sum of |products| times |scales|), ``acc``
    (exact dot product: int64 for INT8, float64 for FP8)."""

    def __init__(self, y, ydbl, bound, acc):
        self.y = y
        self.ydbl = ydbl
        self.bound = bound
        self.acc = acc


def _check(fmt, A, B, sA, sB, block):
    A = _u8(A)
    B = _u8(B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A must be [M,K] and B [N,K]")
    sA = np.ascontiguousarray(np.asarray(sA, np.float32))
    sB = np.ascontiguousarray(np.asarray(sB, np.float32))
    M, K = A.shape
    N = B.shape[0]
    if block:
        if K % 128:
            raise ValueError("Block_FP8 needs K % 128 == 0")
        G = K // 128
        if sA.size != M * G or sB.size != ((N + 127) // 128) * G:
            raise ValueError("block scale shapes")
    else:
        if sA.size != M or sB.size != N:
            raise ValueError("scale shapes")
    if fmt not in (FMT_E4M3, FMT_INT8):
        raise ValueError("fmt")
    return A, B, sA, sB, M, N, K


def scaled_mm(fmt: int, A, sA, B, sB, *, block: bool = False, nthreads: int = 0,
              want_extra: bool = True) -> Result:
    """Y = bf16(scales * (A . B^T)) over every (m, n).

    ``fmt``: FMT_E4M3 or FMT_INT8.  ``A`` [M,K] and ``B`` [N,K] are uint8
    code arrays (int8 arrays are viewed as bytes).  ``sA``/``sB``: fp32
    per-token / per-channel scales, or with ``block=True`` fp32 [M, K/128]
    and [ceil(N/128), K/128] group / block scales.
    """
    A, B, sA, sB, M, N, K = _check(fmt, A, B, sA, sB, block)
    if nthreads <= 0:
        nthreads = os.cpu_count() or 1
    Y = np.zeros((M, N), np.uint16)
    ydbl = np.zeros((M, N), np.float64) if want_extra else None
    bound = np.zeros((M, N), np.float64) if want_extra else None
    acc_i = np.zeros((M, N), np.int64) if (want_extra and fmt == FMT_INT8 and not block) else None
    acc_f = np.zeros((M, N), np.float64) if (want_extra and acc_i is None) else None
    rc = _load().orc_scaled_mm(fmt, int(block), M, N, K, A.ctypes.data, K, sA.ctypes.data,
                               B.ctypes.data, K, sB.ctypes.data, Y.ctypes.data, N,
                               _ptr(ydbl), _ptr(bound), _ptr(acc_i), _ptr(acc_f), nthreads)
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return Result(Y, ydbl, bound, acc_i if acc_i is not None else acc_f)


def scaled_mm_points(fmt: int, A, sA, B, sB, ms, ns, *, block: bool = False,
                     nthreads: int = 0) -> Result:
    """The same definition evaluated only at the positions (ms[i], ns[i])."""
    A, B, sA, sB, M, N, K = _check(fmt, A, B, sA, sB, block)
    pm = np.ascontiguousarray(np.asarray(ms, np.int64))
    pn = np.ascontiguousarray(np.asarray(ns, np.int64))
    n = pm.size
    if pn.size != n:
        raise ValueError("ms and ns differ in length")
    if nthreads <= 0:
        nthreads = os.cpu_count() or 1
    Y = np.zeros(n, np.uint16)
    ydbl = np.zeros(n, np.float64)
    bound = np.zeros(n, np.float64)
    acc_i = np.zeros(n, np.int64) if (fmt == FMT_INT8 and not block) else None
    acc_f = np.zeros(n, np.float64) if acc_i is None else None
    rc = _load().orc_scaled_mm_points(fmt, int(block), M, N, K, A.ctypes.data, K,
                                      sA.ctypes.data, B.ctypes.data, K, sB.ctypes.data,
                                      n, pm.ctypes.data, pn.ctypes.data, Y.ctypes.data,
                                      ydbl.ctypes.data, bound.ctypes.data,
                                      _ptr(acc_i), _ptr(acc_f), nthreads)
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return Result(Y, ydbl, bound, acc_i if acc_i is not None else acc_f)


def _bf16_bits(x) -> np.ndarray:
    """bf16 input as its bit patterns: accepts uint16 bits or float32 values
    that are exactly bf16 (the low 16 bits must be zero)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x)
    f = np.ascontiguousarray(x, np.float32).view(np.uint32)
    if np.any(f & 0xFFFF):
        raise ValueError("input values are not bfloat16")
    return (f >> 16).astype(np.uint16)


def e4m3_nearest(v: float) -> int:
    """Nearest OCP e4m3 code to an fp32 value in [-448, 448], ties to even."""
    return int(_load().orc_e4m3_nearest(float(v)))


def quant_per_token(x, fmt: int):
    """Dynamic per-token quantization of a bf16 activation [M,K]:
    (codes uint8 [M,K], scales fp32 [M]), scale = amax/448 (e4m3) or
    amax/127 (int8), codes = nearest-even of x/scale, clamped."""
    xb = _bf16_bits(x)
    M, K = xb.shape
    q = np.zeros((M, K), np.uint8)
    s = np.zeros(M, np.float32)
    if _load().orc_quant_per_token(fmt, M, K, xb.ctypes.data, K, q.ctypes.data, K,
                                   s.ctypes.data) != 0:
        raise ValueError("oracle rejected its arguments")
    return q, s


def quant_per_group(x, group: int = 128):
    """Per-token-group e4m3 quantization of a bf16 activation [M,K]:
    (codes uint8 [M,K], scales fp32 [M, K/group])."""
    xb = _bf16_bits(x)
    M, K = xb.shape
    q = np.zeros((M, K), np.uint8)
    s = np.zeros((M, K // group), np.float32)
    if _load().orc_quant_per_group(M, K, group, xb.ctypes.data, K, q.ctypes.data, K,
                                   s.ctypes.data) != 0:
        raise ValueError("oracle rejected its arguments")
    return q, s


def rms_norm(x, w, eps: float, residual=None):
    """RMS norm of each row of a bf16 [M,K] activation with bf16 weight [K]:
    y = bf16((h * w) / sqrt(mean(h^2) + eps)) evaluated in double, where
    h = x, or h = bf16(x + residual) when a residual [M,K] is given.
    Returns (y bits [M,K], h bits [M,K] or None)."""
    xb = _bf16_bits(x)
    wb = _bf16_bits(w).ravel()
    M, K = xb.shape
    if wb.size != K:
        raise ValueError("weight must have K elements")
    rb = None if residual is None else _bf16_bits(residual).copy()
    if rb is not None and rb.shape != xb.shape:
        raise ValueError("residual must be [M,K]")
    y = np.zeros((M, K), np.uint16)
    if _load().orc_rms_norm(M, K, xb.ctypes.data, K, _ptr(rb), K, wb.ctypes.data,
                            float(eps), y.ctypes.data, K) != 0:
        raise ValueError("oracle rejected its arguments")
    return y, rb


def silu_and_mul(x):
    """SiLU-and-mul of a bf16 [M, 2K] activation (gate | up):
    y = bf16(g / (1 + exp(-g)) * u) evaluated in double.  Returns y bits [M,K]."""
    xb = _bf16_bits(x)
    M, K2 = xb.shape
    if K2 % 2:
        raise ValueError("the activation must have 2K columns")
    K = K2 // 2
    y = np.zeros((M, K), np.uint16)
    if _load().orc_silu_and_mul(M, K, xb.ctypes.data, K2, y.ctypes.data, K) != 0:
        raise ValueError("oracle rejected its arguments")
    return y


def rms_norm_quant(x, w, eps: float, fmt: int = FMT_E4M3, group: int = 0, residual=None):
    """rms_norm followed by the dynamic quantizer (per token, or per 1 x group
    e4m3 when ``group`` > 0).  Returns (codes, scales, residual out or None)."""
    y, h = rms_norm(x, w, eps, residual)
    q, s = quant_per_group(y, group) if group else quant_per_token(y, fmt)
    return q, s, h


def silu_and_mul_quant(x, fmt: int = FMT_E4M3, group: int = 0):
    """silu_and_mul followed by the dynamic quantizer.  Returns (codes, scales)."""
    y = silu_and_mul(x)
    return quant_per_group(y, group) if group else quant_per_token(y, fmt)


def grouped_scaled_mm(fmt: int, offsets, A, sA, B, sB, *, block: bool = False,
                      max_rows: int | None = None, Y=None, nthreads: int = 0):
    """Grouped (mixture-of-experts) product: for each group g, rows
    offsets[g] .. offsets[g+1]-1 of A / sA times B[g]^T with scales sB[g],
    each exactly the single product on that slice (``scaled_mm``).  Rows of a
    group past ``max_rows`` are not computed: they keep the values of ``Y``
    (bf16 bits [rows, N], zeros when not given).  Returns Y."""
    offsets = np.asarray(offsets, np.int64)
    A = _u8(A)
    B = _u8(B)
    G, N, K = B.shape
    rows = A.shape[0]
    if offsets.shape != (G + 1,) or offsets[0] != 0 or np.any(np.diff(offsets) < 0) or \
            offsets[-1] > rows:
        raise ValueError("offsets must be G+1 nondecreasing row offsets from 0")
    Y = np.zeros((rows, N), np.uint16) if Y is None else np.array(Y, np.uint16, copy=True)
    sA = np.asarray(sA, np.float32)
    sB = np.asarray(sB, np.float32)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if max_rows is not None:
            hi = min(hi, lo + int(max_rows))
        if hi <= lo:
            continue
        r = scaled_mm(fmt, A[lo:hi], sA[lo:hi], B[g], sB[g], block=block, nthreads=nthreads,
                      want_extra=False)
        Y[lo:hi] = r.y
    return Y
