"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the plausible oracle mistake it would catch.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import brute

HERE = os.path.dirname(os.path.abspath(__file__))
FMT = {"fp8": oracle.FMT_E4M3, "int8": oracle.FMT_INT8, "block_fp8": oracle.FMT_E4M3}


def run(case, **kw):
    return oracle.scaled_mm(FMT[case.fmt], case.A, case.sA, case.B, case.sB,
                            block=case.block, **kw)


def bits_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


# --------------------------------------------------------------------------
# e4m3 decode: wrong bias, subnormal rule, sign or NaN codes.
# --------------------------------------------------------------------------
def test_e4m3_decode_matches_torch_cast_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))  # -0 at 0x80


def test_e4m3_spot_values():
    d = oracle.decode_e4m3(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0xFE, 0x7F, 0xFF], np.uint8))
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -9
    assert d[3] == 2.0 ** -6 and d[4] == 7 * 2.0 ** -9 and d[5] == -448.0
    assert np.isnan(d[6]) and np.isnan(d[7])


# --------------------------------------------------------------------------
# bf16 rounding: truncation instead of rounding, ties away from zero,
# double rounding through fp32, flushed subnormals, wrong overflow point.
# --------------------------------------------------------------------------
def _interesting_doubles(g, n):
    xs = []
    # random magnitudes over the whole bf16 range, including subnormals
    e = g.integers(-140, 128, n)
    xs += list(g.uniform(1, 2, n) * np.exp2(e.astype(np.float64)) * g.choice([-1, 1], n))
    # exact ties between two bf16 neighbours and points just off them
    b = g.integers(0x0001, 0x7F7F, n).astype(np.uint16)
    lo = bits_to_f64(b)
    hi = bits_to_f64(b + 1)
    mid = (lo + hi) / 2          # exact in double
    xs += list(mid) + list(np.nextafter(mid, np.inf)) + list(np.nextafter(mid, -np.inf))
    # values that round differently when rounded to fp32 first
    xs += list(mid + (hi - lo) * 2.0 ** -30)
    # around the overflow point and zero
    top = float(bits_to_f64(np.array([0x7F7F], np.uint16))[0])
    xs += [top, top * (1 + 2.0 ** -9), top * (1 + 2.0 ** -8), 2.0 ** 128, -(2.0 ** 128), 0.0, -0.0,
           2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -150]
    return np.array(xs, np.float64)


def test_bf16_rounding_matches_exact_brute_force():
    g = np.random.default_rng(1)
    xs = _interesting_doubles(g, 400)
    ours = oracle.to_bf16_bits(xs)
    for x, o in zip(xs, ours):
        if x == 0:      # a Fraction has no signed zero; +-0 are pinned below
            continue
        assert int(o) == brute.bf16_rne(Fraction(float(x))), x


def test_bf16_rounding_matches_torch_on_fp32_values():
    # On values exactly representable in fp32 one rounding == torch's cast.
    g = np.random.default_rng(2)
    f = g.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_special_values():
    b = oracle.to_bf16_bits(np.array([np.nan, np.inf, -np.inf, -0.0, 1.0, -2.0]))
    assert b[0] & 0x7F80 == 0x7F80 and b[0] & 0x7F
    assert b[1] == 0x7F80 and b[2] == 0xFF80 and b[3] == 0x8000
    assert b[4] == 0x3F80 and b[5] == 0xC000


# --------------------------------------------------------------------------
# The dot products: dropped term, wrong index, transposed operand, wrong
# decode in the inner loop, integer overflow.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_tiny_shapes_equal_exact_rational_brute_force(fmt):
    K = 256 if fmt == "block_fp8" else 48
    N = 256 if fmt == "block_fp8" else 5          # two weight blocks along N
    case = synth.make_case(fmt, 3, N, K, outliers=True, root=11)
    r = run(case)
    y, acc = brute.gemm_exact(fmt, case.A, case.sA, case.B, case.sB, block=case.block)
    cols = range(N) if N <= 8 else [0, 1, 127, 128, 255]
    for m in range(3):
        for n in cols:
            assert Fraction(int(r.acc[m, n])) == acc[m][n] if fmt == "int8" \
                else Fraction(float(r.acc[m, n])) == acc[m][n]
            # y before rounding: within a few double roundings of the exact value
            assert abs(Fraction(float(r.ydbl[m, n])) - y[m][n]) <= abs(y[m][n]) * Fraction(1, 2 ** 50)
            assert int(r.y[m, n]) == brute.bf16_rne(y[m][n]), (m, n)


def test_int8_dot_equals_numpy_int64_matmul():
    case = synth.make_case("int8", 24, 300, 2048, root=5)
    r = run(case)
    ref = case.A.view(np.int8).astype(np.int64) @ case.B.view(np.int8).astype(np.int64).T
    assert np.array_equal(r.acc, ref)


@pytest.mark.parametrize("K", [1024, 6144])
def test_fp8_dot_equals_float64_matmul_of_torch_decoded_values(K):
    # Every partial sum is exact in double, so any summation order agrees bit for bit.
    case = synth.make_case("fp8", 16, 256, K, outliers=True, root=6)
    r = run(case)
    a = torch.from_numpy(case.A).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    b = torch.from_numpy(case.B).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(r.acc, a @ b.T)


def test_exhaustive_code_pairs():
    # One non-zero per row: acc[m,n] = dec(code m) * dec(code n) for every pair.
    for fmt in ("fp8", "int8"):
        codes = np.arange(256, dtype=np.uint8)
        if fmt == "fp8":
            codes = codes[(codes & 0x7F) != 0x7F]          # drop the two NaN codes
        K = 16
        A = np.zeros((codes.size, K), np.uint8)
        A[:, 0] = codes
        B = A.copy()
        ones = np.ones(codes.size, np.float32)
        r = oracle.scaled_mm(FMT[fmt], A, ones, B, ones)
        if fmt == "fp8":
            v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        else:
            v = codes.view(np.int8).astype(np.float64)
        assert np.array_equal(np.asarray(r.acc, np.float64), np.outer(v, v))
        ref_bits = torch.from_numpy(np.outer(v, v).astype(np.float32)).to(torch.bfloat16) \
            .view(torch.int16).numpy().view(np.uint16)     # products are exact in fp32
        # a sum with +0 terms is +0 while 0 * (-x) alone is -0: zeros compare by value
        zero = (ref_bits & 0x7FFF) == 0
        assert np.array_equal(r.y[~zero], ref_bits[~zero])
        assert ((r.y[zero] & 0x7FFF) == 0).all()


# --------------------------------------------------------------------------
# Scale application: scale dropped, applied twice, taken from the wrong row,
# block index off by one, groups paired with the wrong scales.
# --------------------------------------------------------------------------
def test_golden_worked_examples():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        K, M, N = c["K"], c["M"], c["N"]
        if "A" in c:
            A = np.array(c["A"], np.int64).astype(np.int8).view(np.uint8) if c["fmt"] == "int8" \
                else np.array(c["A"], np.uint8)
            B = np.array(c["B"], np.int64).astype(np.int8).view(np.uint8) if c["fmt"] == "int8" \
                else np.array(c["B"], np.uint8)
        else:
            A = np.zeros((M, K), np.uint8)
            for (lo, hi, code) in c["A_rows"][0]["fill"]:
                A[0, lo:hi] = code
            B = np.zeros((N, K), np.uint8)
            for (lo, hi, code) in c["B_rows_all"]["fill"]:
                B[:, lo:hi] = code
        r = oracle.scaled_mm(FMT[c["fmt"]], A, np.array(c["sA"], np.float32), B,
                             np.array(c["sB"], np.float32), block=c["block"])
        if "Y_bits" in c:
            assert r.y.tolist() == c["Y_bits"], c["name"]
            assert np.asarray(r.acc, np.float64).tolist() == np.asarray(c["acc"], np.float64).tolist()
        else:
            assert (r.y == c["Y_bits_all"]).all(), c["name"]
            assert (r.acc == c["acc_all"]).all()


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_constant_operands_closed_form(fmt):
    K, M, N = 1024, 4, 8
    ca, cb = (0x44, 0xB2) if fmt == "fp8" else (3, 0xF9)   # 3.0, -0.625 | 3, -7
    A = np.full((M, K), ca, np.uint8)
    B = np.full((N, K), cb, np.uint8)
    sA = np.array([0.5, 0.25, 2.0, 1.5], np.float32)
    sB = np.linspace(0.01, 0.08, N).astype(np.float32)
    r = oracle.scaled_mm(FMT[fmt], A, sA, B, sB)
    if fmt == "fp8":
        da, db = 3.0, -0.625
    else:
        da, db = 3.0, -7.0
    for m in range(M):
        for n in range(N):
            exact = Fraction(K) * Fraction(da) * Fraction(db) * Fraction(float(sA[m])) * Fraction(float(sB[n]))
            assert int(r.y[m, n]) == brute.bf16_rne(exact)


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_power_of_two_scale_homogeneity(fmt):
    case = synth.make_case(fmt, 6, 128, 512, root=7)
    r0 = run(case)
    for j in (-3, 5):
        c2 = synth.Case(case.fmt, case.M, case.N, case.K, case.A,
                        (case.sA * np.float32(2.0 ** j)).astype(np.float32), case.B, case.sB)
        r1 = run(c2)
        assert np.array_equal(bits_to_f64(r1.y), bits_to_f64(r0.y) * 2.0 ** j)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_sign_symmetry(fmt):
    case = synth.make_case(fmt, 5, 64, 512, root=8)
    neg = (case.A ^ 0x80) if fmt == "fp8" else (-case.A.view(np.int8)).astype(np.int8).view(np.uint8)
    r0 = run(case)
    r1 = oracle.scaled_mm(FMT[fmt], neg, case.sA, case.B, case.sB)
    nz = r0.y & 0x7FFF != 0
    assert np.array_equal(r1.y[nz], r0.y[nz] ^ 0x8000)


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_identity_weights(fmt):
    K = 256
    case = synth.make_case(fmt, 7, K, K, root=9)
    one = 1 if fmt == "int8" else 0x38
    B = np.zeros((K, K), np.uint8)
    B[np.arange(K), np.arange(K)] = one
    if fmt == "block_fp8":
        sB = np.ones((K // 128, K // 128), np.float32)
        r = oracle.scaled_mm(FMT[fmt], case.A, case.sA, B, sB, block=True)
        scale_a = np.repeat(case.sA, 128, axis=1)           # sA[m, n // 128]
    else:
        sB = np.ones(K, np.float32)
        r = oracle.scaled_mm(FMT[fmt], case.A, case.sA, B, sB)
        scale_a = np.repeat(case.sA[:, None], K, axis=1)
    if fmt == "int8":
        dec = case.A.view(np.int8).astype(np.float64)
    else:
        dec = torch.from_numpy(case.A).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for m in range(7):
        for n in range(0, K, 17):
            exact = Fraction(float(dec[m, n])) * Fraction(float(scale_a[m, n]))
            assert int(r.y[m, n]) == brute.bf16_rne(exact)


def test_block_with_uniform_scales_equals_token_channel():
    M, N, K = 5, 256, 512
    case = synth.make_case("fp8", M, N, K, root=10)
    sA_blk = np.repeat(case.sA[:, None], K // 128, axis=1)
    sB_pc = np.full(N, np.float32(0.0123))
    sB_blk = np.full((N // 128, K // 128), np.float32(0.0123))
    r_tc = oracle.scaled_mm(oracle.FMT_E4M3, case.A, case.sA, case.B, sB_pc)
    r_bl = oracle.scaled_mm(oracle.FMT_E4M3, case.A, sA_blk, case.B, sB_blk, block=True)
    # the exact products agree; the rounded outputs agree except where the two
    # double-rounding orders straddle a bf16 midpoint (checked against exact).
    assert np.array_equal(r_tc.acc, r_bl.acc)
    diff = np.argwhere(r_tc.y != r_bl.y)
    assert len(diff) <= 2


# --------------------------------------------------------------------------
# Algebraic identities of the variants: K partition (Split-K) and transpose
# (Swap-AB), both stated in the pages' "Kernel Implementation" section.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_k_partition_identity(fmt):
    case = synth.make_case(fmt, 9, 96, 1024, root=12)
    full = run(case).acc
    parts = 0
    for lo, hi in ((0, 256), (256, 640), (640, 1024)):
        rp = oracle.scaled_mm(FMT[fmt], np.ascontiguousarray(case.A[:, lo:hi]), case.sA,
                              np.ascontiguousarray(case.B[:, lo:hi]), case.sB)
        parts = parts + rp.acc
    assert np.array_equal(full, parts)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_transpose_identity(fmt):
    case = synth.make_case(fmt, 9, 40, 512, root=13)
    r = run(case)
    rt = oracle.scaled_mm(FMT[fmt], case.B, case.sB, case.A, case.sA)
    assert np.array_equal(r.acc, rt.acc.T)
    assert np.array_equal(r.y, rt.y.T)


def test_bound_matrix():
    case = synth.make_case("fp8", 8, 64, 512, root=14)
    r = run(case)
    assert (r.bound >= np.abs(r.ydbl) * (1 - 1e-12)).all()
    # all-positive operands: no cancellation, so the bound equals |y|
    A = case.A & 0x7F
    B = case.B & 0x7F
    r2 = oracle.scaled_mm(oracle.FMT_E4M3, A, case.sA, B, case.sB)
    assert np.allclose(r2.bound, r2.ydbl, rtol=1e-14, atol=0)


# --------------------------------------------------------------------------
# The bound matrix S (the scale of the elementwise FP8 / Block_FP8 rule):
# |sum ab| in place of sum |ab|, a missing |.| on a scale, a Block bound
# paired with the wrong group or weight block row, a constant factor.
# --------------------------------------------------------------------------
def _abs_decoded(fmt, codes):
    """|value| of each code, decoded by torch's casts (not by the oracle)."""
    c = np.ascontiguousarray(codes).view(np.uint8)
    if fmt == "int8":
        return np.abs(c.view(np.int8).astype(np.int64))
    return np.abs(torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy())


def _tiny_mixed_case(fmt, M, N, K, seed):
    """Random codes of both signs (no NaN codes) and scales of both signs."""
    g = np.random.default_rng(seed)
    if fmt == "int8":
        A = g.integers(-128, 128, (M, K)).astype(np.int8).view(np.uint8)
        B = g.integers(-128, 128, (N, K)).astype(np.int8).view(np.uint8)
    else:
        A = (g.integers(0, 0x7F, (M, K)) | (g.integers(0, 2, (M, K)) << 7)).astype(np.uint8)
        B = (g.integers(0, 0x7F, (N, K)) | (g.integers(0, 2, (N, K)) << 7)).astype(np.uint8)
    if fmt == "block_fp8":
        sA = (g.uniform(0.01, 2, (M, K // 128)) * g.choice([-1, 1], (M, K // 128))).astype(np.float32)
        sB = (g.uniform(0.01, 2, (N // 128, K // 128)) * g.choice([-1, 1], (N // 128, K // 128))
              ).astype(np.float32)
    else:
        sA = (g.uniform(0.01, 2, M) * g.choice([-1, 1], M)).astype(np.float32)
        sB = (g.uniform(0.01, 2, N) * g.choice([-1, 1], N)).astype(np.float32)
    return A, sA, B, sB


@pytest.mark.parametrize("fmt,M,N,K", [("fp8", 3, 5, 48), ("int8", 3, 5, 48),
                                       ("block_fp8", 2, 256, 256)])
def test_bound_matrix_exact_rationals(fmt, M, N, K):
    A, sA, B, sB = _tiny_mixed_case(fmt, M, N, K, seed=17)
    block = fmt == "block_fp8"
    r = oracle.scaled_mm(FMT[fmt], A, sA, B, sB, block=block)
    # Block: a few outputs on each side of the weight-block boundary at n = 128
    cols = (0, 1, 127, 128, 200, 255) if block else range(N)
    for m in range(M):
        for n in cols:
            if block:
                nb = n // 128
                exact = brute.bound_exact(fmt, A[m:m + 1], sA[m:m + 1], B[n:n + 1],
                                          sB[nb:nb + 1], block=True)[0][0]
            else:
                exact = brute.bound_exact(fmt, A[m:m + 1], sA[m:m + 1], B[n:n + 1],
                                          sB[n:n + 1])[0][0]
            got = Fraction(float(r.bound[m, n]))
            assert abs(got - exact) <= exact * Fraction(1, 2 ** 50), (fmt, m, n, float(exact), float(got))
    # cancellation really happens in these inputs: the bound exceeds |y| by a wide margin somewhere
    assert (r.bound > 2 * np.abs(r.ydbl)).any()


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_bound_matrix_numpy(fmt):
    # The workloads' value distributions at a size spanning several weight
    # blocks; S recomputed from torch-decoded magnitudes with numpy products.
    # Every e4m3 product is a multiple of 2^-18 and every int8 product an
    # integer, so the sums of magnitudes are exact in float64 in any order and
    # the scaling is the same two roundings in the same order: bit-exact.
    case = synth.make_case(fmt, 12, 384, 1024, root=18)
    r = run(case)
    a, b = _abs_decoded(fmt, case.A), _abs_decoded(fmt, case.B)
    if fmt != "block_fp8":
        P = (a.astype(np.float64) @ b.astype(np.float64).T)
        S = (P * np.abs(case.sA.astype(np.float64))[:, None]) * np.abs(case.sB.astype(np.float64))[None, :]
    else:
        G = case.K // 128
        S = np.zeros((case.M, case.N))
        nb = np.arange(case.N) // 128
        for g in range(G):
            P = a[:, g * 128:(g + 1) * 128] @ b[:, g * 128:(g + 1) * 128].T
            sa = np.abs(case.sA[:, g].astype(np.float64))[:, None]
            sb = np.abs(case.sB[nb, g].astype(np.float64))[None, :]
            S = S + (P * sa) * sb
    assert np.array_equal(r.bound, S)


def test_bound_matrix_block_all_positive_equals_y():
    # Block_FP8 with positive codes and scales: no cancellation anywhere, so S == y
    case = synth.make_case("block_fp8", 5, 256, 512, root=19)
    A = case.A & 0x7F
    B = case.B & 0x7F
    r = oracle.scaled_mm(oracle.FMT_E4M3, A, case.sA, B, case.sB, block=True)
    assert np.array_equal(r.bound, r.ydbl)
    # ... and flipping the sign of one operand's codes leaves S unchanged
    r2 = oracle.scaled_mm(oracle.FMT_E4M3, A | 0x80, case.sA, B, case.sB, block=True)
    assert np.array_equal(r2.bound, r.bound)
    assert np.array_equal(r2.ydbl, -r.ydbl)


def test_bound_golden_cancellation():
    with open(os.path.join(HERE, "golden", "bound_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        M, N, K = c["M"], c["N"], c["K"]
        A = np.zeros((M, K), np.int64)
        for row, k, code in c["A"]:
            A[row, k] = code
        B = np.zeros((N, K), np.int64)
        if "B" in c:
            for row, k, code in c["B"]:
                B[row, k] = code
        else:
            for k, code in c["B_all_rows"]:
                B[:, k] = code
        A = A.astype(np.int8).view(np.uint8) if c["fmt"] == "int8" else A.astype(np.uint8)
        B = B.astype(np.int8).view(np.uint8) if c["fmt"] == "int8" else B.astype(np.uint8)
        r = oracle.scaled_mm(FMT[c["fmt"]], A, np.array(c["sA"], np.float32), B,
                             np.array(c["sB"], np.float32), block=c["block"])
        if "S" in c:
            assert r.bound.tolist() == c["S"], c["name"]
            assert r.ydbl.tolist() == c["y"], c["name"]
        else:
            for blk, (yv, sv) in enumerate(zip(c["y_by_block"], c["S_by_block"])):
                cols = slice(blk * 128, (blk + 1) * 128)
                assert (r.bound[:, cols] == sv).all(), (c["name"], blk)
                assert (r.ydbl[:, cols] == yv).all(), (c["name"], blk)


def test_points_mode_equals_full():
    case = synth.make_case("block_fp8", 7, 256, 512, root=15)
    full = run(case)
    g = np.random.default_rng(3)
    ms = g.integers(0, 7, 50)
    ns = g.integers(0, 256, 50)
    pts = oracle.scaled_mm_points(oracle.FMT_E4M3, case.A, case.sA, case.B, case.sB, ms, ns, block=True)
    assert np.array_equal(pts.y, full.y[ms, ns])
    assert np.array_equal(pts.acc, full.acc[ms, ns])


def test_int8_extreme_accumulator_is_exact():
    # K = 25600 rows of -128 * -128: 419430400 < 2^31; int64 in the oracle.
    K = 25600
    A = np.full((1, K), 0x80, np.uint8)
    B = np.full((2, K), 0x80, np.uint8)
    B[1] = 0x7F
    r = oracle.scaled_mm(oracle.FMT_INT8, A, np.ones(1, np.float32), B, np.ones(2, np.float32))
    assert r.acc.tolist() == [[K * 128 * 128, -K * 128 * 127]]


def test_degenerate_sizes():
    A = np.zeros((0, 32), np.uint8)
    B = np.zeros((4, 32), np.uint8)
    r = oracle.scaled_mm(oracle.FMT_E4M3, A, np.ones(0, np.float32), B, np.ones(4, np.float32))
    assert r.y.shape == (0, 4)
