"""Pins of the oracle's fused producers (CPU only): RMS norm and SiLU-and-mul
ahead of the dynamic quantizer.

The producers are named in "HelionがvLLMに統合 ..." (24-ai.news), section
"vLLMに統合されたカーネル", items 2, 3, 6 and 7; the pages give no formula.
The reading pinned here: the bf16 output of the producer is its real-number
value rounded once to nearest-even, and the fused kernel returns what the
quantizer returns on that bf16 activation.

The reference below is independent of the C oracle: exact rationals
(fractions.Fraction) for sums, squares and products, 60-digit decimal
arithmetic for the square root and the exponential, and a bf16 rounding
written over exact rationals.  Each test names the plausible mistake it
would catch.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import oracle

getcontext().prec = 60


def bf16_bits(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def random_bf16(g, shape, scale=1.0):
    return bits_to_f(bf16_bits((g.standard_normal(shape) * scale).astype(np.float32)))


def bf16_exact(v: Fraction):
    """Nearest-even bf16 of an exact rational -> (bits of |v| with sign of v,
    distance of v from the nearest rounding tie in units of the bf16 spacing)."""
    neg = v < 0
    a = -v if neg else v
    if a == 0:
        return (0x8000 if neg else 0), Fraction(1, 2)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                                   # subnormal spacing below 2^-126
    ulp = Fraction(2) ** (e - 7)
    q = a / ulp
    n = q.numerator // q.denominator
    frac = q - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = np.float32(float(n * ulp))
    assert Fraction(float(val)) == n * ulp
    b = int(np.array([val], np.float32).view(np.uint32)[0] >> 16)
    return (b | 0x8000) if neg else b, abs(frac - Fraction(1, 2))


def dec_to_frac(d: Decimal) -> Fraction:
    return Fraction(d)


def rms_reference(x, w, eps, residual=None):
    """Exact-rational / 60-digit reference of the RMS norm, returning the bf16
    bits and the smallest distance to a tie seen."""
    M, K = x.shape
    y = np.zeros((M, K), np.uint16)
    hout = np.zeros((M, K), np.uint16)
    closest = Fraction(1, 2)
    for m in range(M):
        h = []
        for k in range(K):
            v = Fraction(float(x[m, k]))
            if residual is not None:
                hb, _ = bf16_exact(v + Fraction(float(residual[m, k])))   # exact: ties decided exactly
                hout[m, k] = hb
                v = Fraction(float(bits_to_f(np.array([hb]))[0]))
            h.append(v)
        ms = sum(t * t for t in h) / K + Fraction(float(np.float32(eps)))
        inv = dec_to_frac(1 / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt())
        for k in range(K):
            yb, d = bf16_exact(h[k] * Fraction(float(w[k])) * inv)
            closest = min(closest, d)
            y[m, k] = yb
    return y, hout, closest


def silu_reference(x):
    M, K2 = x.shape
    K = K2 // 2
    y = np.zeros((M, K), np.uint16)
    closest = Fraction(1, 2)
    for m in range(M):
        for k in range(K):
            g = Decimal(float(x[m, k]))
            u = Fraction(float(x[m, K + k]))
            s = dec_to_frac(g / (1 + (-g).exp()))
            yb, d = bf16_exact(s * u)
            closest = min(closest, d)
            y[m, k] = yb
    return y, closest


# --------------------------------------------------------------------------
# RMS norm against the exact reference: a mean over K-1, eps outside the
# square root or added to the root, the weight applied to h^2, a missing
# weight, the wrong rounding of the output.
# --------------------------------------------------------------------------
def test_rms_norm_matches_exact_reference():
    g = np.random.default_rng(11)
    for (M, K, eps, sc) in [(3, 8, 1e-6, 1.0), (2, 37, 1e-5, 0.01), (2, 64, 0.0, 30.0),
                            (1, 5, 0.5, 0.3)]:
        x = random_bf16(g, (M, K), sc)
        w = random_bf16(g, (K,), 1.0)
        want, _, closest = rms_reference(x, w, eps)
        got, _ = oracle.rms_norm(x, w, eps)
        assert closest > Fraction(1, 10 ** 9)          # no case rests on a near tie
        assert np.array_equal(got, want), (M, K, eps)


def test_rms_norm_with_residual_matches_exact_reference():
    # catches: the norm taken over x instead of x + r, the sum not rounded to
    # bf16 before the norm, the residual not replaced by the sum
    g = np.random.default_rng(12)
    x = random_bf16(g, (3, 24), 1.0)
    r = random_bf16(g, (3, 24), 3.0)
    w = random_bf16(g, (24,), 0.5)
    want, want_h, closest = rms_reference(x, w, 1e-6, residual=r)
    got, got_h = oracle.rms_norm(x, w, 1e-6, residual=r)
    assert closest > Fraction(1, 10 ** 9)
    assert np.array_equal(got_h, want_h)
    assert np.array_equal(got, want)


def test_rms_norm_residual_zero_is_plain_norm():
    g = np.random.default_rng(13)
    x = random_bf16(g, (4, 40))
    w = random_bf16(g, (40,))
    y0, _ = oracle.rms_norm(x, w, 1e-6)
    y1, h = oracle.rms_norm(x, w, 1e-6, residual=np.zeros_like(x))
    assert np.array_equal(y0, y1)
    assert np.array_equal(h, bf16_bits(x))


def test_rms_norm_scale_invariance_without_eps():
    # with eps = 0 the norm of 2^j x equals the norm of x bit for bit (the
    # square root of 4^j is exact); catches a missing square root, a sum of
    # |h| instead of h^2, a division by K^2
    g = np.random.default_rng(14)
    x = random_bf16(g, (5, 48))
    w = random_bf16(g, (48,))
    y, _ = oracle.rms_norm(x, w, 0.0)
    for j in (-20, -1, 3, 9):
        ys, _ = oracle.rms_norm(x * np.float32(2.0 ** j), w, 0.0)
        assert np.array_equal(ys, y), j


def test_rms_norm_permutation_equivariance():
    # a permutation of the columns (with the weight permuted alike) permutes
    # the output: catches a weight indexed by the wrong k, a row stride bug
    g = np.random.default_rng(15)
    x = random_bf16(g, (3, 33))
    w = random_bf16(g, (33,))
    p = g.permutation(33)
    y, _ = oracle.rms_norm(x, w, 1e-6)
    yp, _ = oracle.rms_norm(np.ascontiguousarray(x[:, p]), w[p], 1e-6)
    assert np.array_equal(yp, y[:, p])


def test_rms_norm_closed_forms():
    # K = 1 or a constant row with eps = 0: y = sign(x) * w exactly
    g = np.random.default_rng(16)
    w = random_bf16(g, (1,))
    for v in (3.0, -0.125, 1e-3, 7e4):
        xb = bits_to_f(bf16_bits(np.array([[v]], np.float32)))
        y, _ = oracle.rms_norm(xb, w, 0.0)
        assert y[0, 0] == bf16_bits(np.sign(xb[0, 0]) * w)[0]
    x = np.full((1, 16), -2.5, np.float32)
    w16 = random_bf16(g, (16,))
    y, _ = oracle.rms_norm(x, w16, 0.0)
    assert np.array_equal(y[0], bf16_bits(-w16))
    # x = [3, 4], w = 1: y = [3, 4] / sqrt(12.5) -> bf16 0.84765625, 1.1328125
    y, _ = oracle.rms_norm(np.array([[3.0, 4.0]], np.float32), np.ones(2, np.float32), 0.0)
    assert list(bits_to_f(y[0])) == [0.84765625, 1.1328125]


# --------------------------------------------------------------------------
# SiLU-and-mul: exp(g) for exp(-g), gate and up swapped, the product taken
# on the rounded SiLU, a lost sign.
# --------------------------------------------------------------------------
def test_silu_and_mul_matches_exact_reference():
    g = np.random.default_rng(21)
    for (M, K, sc) in [(3, 16, 1.0), (2, 40, 4.0), (2, 8, 0.02)]:
        x = random_bf16(g, (M, 2 * K), sc)
        want, closest = silu_reference(x)
        got = oracle.silu_and_mul(x)
        assert closest > Fraction(1, 10 ** 9)
        assert np.array_equal(got, want), (M, K)


def test_silu_and_mul_special_values():
    gate = np.array([0.0, 64.0, -1000.0, 1.0, -1.0, 2.0], np.float32)
    up = np.array([3.0, 0.5, 2.0, 0.0, 1.0, -1.0], np.float32)
    y = bits_to_f(oracle.silu_and_mul(np.concatenate([gate, up])[None, :]))[0]
    assert y[0] == 0.0                                   # silu(0) = 0
    assert y[1] == 32.0                                  # silu(64) = 64 to double precision
    assert y[2] == 0.0 and np.signbit(y[2])              # silu(-1000) * 2 = -0
    assert y[3] == 0.0                                   # up = 0
    # silu(-1) = -1 / (1 + e) = -0.26894...; silu(2) * -1 = -1.76159...
    assert y[4] == np.float32(-0.26953125) and y[5] == np.float32(-1.7578125)


def test_fused_oracle_is_the_composition():
    g = np.random.default_rng(22)
    x = random_bf16(g, (4, 256))
    w = random_bf16(g, (256,))
    y, _ = oracle.rms_norm(x, w, 1e-6)
    q, s, _ = oracle.rms_norm_quant(x, w, 1e-6, oracle.FMT_INT8)
    q2, s2 = oracle.quant_per_token(y, oracle.FMT_INT8)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    q, s = oracle.silu_and_mul_quant(x, group=128)
    q2, s2 = oracle.quant_per_group(oracle.silu_and_mul(x), 128)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
