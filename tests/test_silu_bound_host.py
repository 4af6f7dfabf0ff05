"""The bound behind the spread SiLU-and-mul rows (k_silu_spread).

Every workgroup of a row finds the row's maximum |value| itself: values
whose bound max(g, 0.279) * |u| is below the maximum m of its own exact
values are skipped, which is exact only if the bound is never below
|silu(g) * u|.  Checked here for every finite bf16 gate (all 65536 bit
patterns but inf / NaN), with the real value silu(g) = g / (1 + e^-g) in
double, and the fp32 product the kernel forms for the bound checked against
the exact bound for the up values where rounding could matter.
"""
import numpy as np


def all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def silu(g):
    g = g.astype(np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def test_bound_covers_every_bf16_gate():
    g = all_bf16()
    s = np.abs(silu(g))
    b = np.maximum(g.astype(np.float64), np.float64(np.float32(0.279)))
    assert np.all(s <= b), g[s > b][:5]
    # the two regimes the bound rests on, with their margins
    pos = g > 0
    assert np.all(s[pos] <= g[pos].astype(np.float64))   # equal only where double rounds
    assert np.abs(silu(g[~pos])).max() < 0.2785 < np.float32(0.279)


def test_fp32_bound_is_not_below_the_exact_bound():
    # fl32(max(g, 0.279f) * |u|) over every bf16 gate and a spread of bf16 up
    # values (products of two bf16 numbers are exact in fp32; 0.279f times a
    # bf16 value may round down by half an ulp, still above 0.2785 |u|)
    g = all_bf16()
    u = all_bf16()[::97]
    u = u[(np.abs(u) > 2.0 ** -60) & (np.abs(u) < 2.0 ** 60)]
    gm = np.maximum(g, np.float32(0.279)).astype(np.float32)
    for uu in u:
        b32 = (gm * np.float32(abs(uu))).astype(np.float64)
        exact = np.abs(silu(g)) * abs(float(uu))
        ok = (b32 >= exact) | ~np.isfinite(b32) | (b32 < 2.0 ** -100)
        assert ok.all(), (uu, g[~ok][:5])
