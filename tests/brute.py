"""Exact-rational brute force used to pin the oracle on tiny inputs.

Independent of the oracle: code values come from torch's e4m3 / bf16 casts
(library routines) turned into exact Fractions, and rounding to bf16 is done
by searching the sorted table of every finite bf16 value for the nearest
one, ties going to the even bit pattern.
"""
from __future__ import annotations

import bisect
from fractions import Fraction
from functools import lru_cache

import numpy as np
import torch


@lru_cache(maxsize=1)
def e4m3_table():
    """code -> Fraction (None for NaN), from torch's float8_e4m3fn cast."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float32).tolist()
    return [None if v != v else Fraction(v) for v in vals]


def int8_value(code: int) -> Fraction:
    return Fraction(int(np.uint8(code).view(np.int8)))


@lru_cache(maxsize=1)
def _bf16_positive():
    """Sorted (value, bits) of every positive finite bf16, plus 2^128 for +inf."""
    bits = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float64).tolist()
    table = [(Fraction(v), b) for b, v in enumerate(vals)]
    table.append((Fraction(2) ** 128, 0x7F80))
    keys = [t[0] for t in table]
    return table, keys


def bf16_rne(v: Fraction) -> int:
    """Exact value -> bf16 bits, nearest, ties to the even bit pattern."""
    table, keys = _bf16_positive()
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    if a >= keys[-1]:
        return sign | 0x7F80
    i = bisect.bisect_left(keys, a)
    if keys[i] == a:
        return sign | table[i][1]
    lo, hi = table[i - 1], table[i]
    dlo, dhi = a - lo[0], hi[0] - a
    if dlo < dhi:
        pick = lo[1]
    elif dhi < dlo:
        pick = hi[1]
    else:
        pick = lo[1] if lo[1] % 2 == 0 else hi[1]
    return sign | pick


def decode(fmt: str, code: int) -> Fraction:
    return int8_value(code) if fmt == "int8" else e4m3_table()[code]


def gemm_exact(fmt: str, A, sA, B, sB, block: bool = False):
    """Exact y[m][n] as Fractions and the exact dot products."""
    A = np.asarray(A).view(np.uint8)
    B = np.asarray(B).view(np.uint8)
    M, K = A.shape
    N = B.shape[0]
    y = [[None] * N for _ in range(M)]
    acc = [[None] * N for _ in range(M)]
    da = [[decode(fmt, int(c)) for c in row] for row in A]
    db = [[decode(fmt, int(c)) for c in row] for row in B]
    for m in range(M):
        for n in range(N):
            if not block:
                s = sum((da[m][k] * db[n][k] for k in range(K)), Fraction(0))
                acc[m][n] = s
                y[m][n] = s * Fraction(float(sA[m])) * Fraction(float(sB[n]))
            else:
                G = K // 128
                tot = Fraction(0)
                ysum = Fraction(0)
                for g in range(G):
                    p = sum((da[m][k] * db[n][k] for k in range(g * 128, g * 128 + 128)),
                            Fraction(0))
                    tot += p
                    ysum += p * Fraction(float(sA[m][g])) * Fraction(float(sB[n // 128][g]))
                acc[m][n] = tot
                y[m][n] = ysum
    return y, acc


def bound_exact(fmt: str, A, sA, B, sB, block: bool = False):
    """Exact bound matrix S[m][n] as Fractions: the sum over k of
    |a[m,k] b[n,k]| times |sA[m]| |sB[n]| (token / channel scales), or for
    1x128 / 128x128 block scales the sum over K groups g of
    |sA[m,g]| |sB[n//128,g]| times the group's sum of |a b|."""
    A = np.asarray(A).view(np.uint8)
    B = np.asarray(B).view(np.uint8)
    M, K = A.shape
    N = B.shape[0]
    da = [[abs(decode(fmt, int(c))) for c in row] for row in A]
    db = [[abs(decode(fmt, int(c))) for c in row] for row in B]
    S = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            if not block:
                s = sum((da[m][k] * db[n][k] for k in range(K)), Fraction(0))
                S[m][n] = s * abs(Fraction(float(sA[m]))) * abs(Fraction(float(sB[n])))
            else:
                tot = Fraction(0)
                for g in range(K // 128):
                    p = sum((da[m][k] * db[n][k] for k in range(g * 128, g * 128 + 128)),
                            Fraction(0))
                    tot += p * abs(Fraction(float(sA[m][g]))) * abs(Fraction(float(sB[n // 128][g])))
                S[m][n] = tot
    return S
