"""Pins of the oracle's activation quantizers (CPU only).

The quantizers are restated from the kernel list of "HelionがvLLMに統合 ..."
(24-ai.news), section "vLLMに統合されたカーネル", items 1 and 5 (dynamic
per-token FP8 and per-token-group FP8 quantization), with the scale rule
amax/448 (amax/127 for int8).  Each test names the plausible mistake it
would catch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def bf16_bits(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def e4m3_values():
    codes = np.arange(0x7F, dtype=np.uint8)          # +0 .. 448
    return codes, torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()


# --------------------------------------------------------------------------
# Nearest-e4m3 rounding: wrong tie rule, off-by-one code, lost sign of zero,
# wrong subnormal spacing, no saturation.
# --------------------------------------------------------------------------
def test_e4m3_nearest_round_trips_every_code():
    codes, vals = e4m3_values()
    for c, v in zip(codes, vals):
        assert oracle.e4m3_nearest(float(v)) == c
        if v != 0:
            assert oracle.e4m3_nearest(float(-v)) == (int(c) | 0x80)
    assert oracle.e4m3_nearest(-0.0) == 0x80


def test_e4m3_nearest_ties_go_to_even_code():
    codes, vals = e4m3_values()
    for c in range(0x7E):
        lo, hi = float(vals[c]), float(vals[c + 1])
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2                    # midpoint exact in fp32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_nearest(float(mid)) == want, (c, lo, hi)
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1000))
        assert oracle.e4m3_nearest(float(below)) == c
        assert oracle.e4m3_nearest(float(above)) == c + 1


def test_e4m3_nearest_matches_torch_cast_on_random_values():
    g = np.random.default_rng(5)
    v = np.concatenate([g.uniform(-448, 448, 4000), g.uniform(-0.05, 0.05, 4000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_nearest(float(x)) for x in v], np.uint8)
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------
# Whole quantizers against the independent numpy/torch quantizer that makes
# the GEMM inputs: wrong amax, scale formula or per-row/group indexing.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("outliers", [False, True])
def test_per_token_matches_numpy_quantizer(fmt, outliers):
    x = synth.activations(37, 2048 + 64, (0, 2, 37, 2112), outliers=outliers, outlier_key=(0, 3, 2112))
    q, s = oracle.quant_per_token(x, oracle.FMT_INT8 if fmt == "int8" else oracle.FMT_E4M3)
    q_ref, s_ref = synth.quant_rows(x, fmt)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_per_group_matches_numpy_quantizer():
    x = synth.activations(19, 1024, (0, 2, 19, 1024), outliers=True, outlier_key=(0, 3, 1024))
    q, s = oracle.quant_per_group(x, 128)
    q_ref, s_ref = synth.quant_groups(x, 128)
    assert s.shape == (19, 8)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_per_group_scales_are_local_to_each_group():
    # one large value in group 1 only: groups 0 and 2 keep their own scale
    x = np.full((1, 384), 0.5, np.float32)
    x[0, 200] = 64.0
    q, s = oracle.quant_per_group(x, 128)
    assert s[0, 0] == np.float32(0.5) / np.float32(448)
    assert s[0, 1] == np.float32(64.0) / np.float32(448)
    assert s[0, 2] == s[0, 0]
    assert q[0, 0] == 0x7E and q[0, 200] == 0x7E and q[0, 300] == 0x7E


# --------------------------------------------------------------------------
# Closed forms: scale from the row maximum, ties to even for int8, clamping,
# zero rows.
# --------------------------------------------------------------------------
def test_int8_half_ties_round_to_even():
    row = np.array([[127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 126.5, -127.0]], np.float32)
    q, s = oracle.quant_per_token(row, oracle.FMT_INT8)
    assert s[0] == np.float32(1.0)
    assert q[0].view(np.int8).tolist() == [127, 2, 4, -2, 0, 0, 126, -127]


def test_e4m3_row_with_amax_448_keeps_its_codes():
    codes, vals = e4m3_values()
    row = np.concatenate([vals, -vals[1:]])[None, :].astype(np.float32)   # amax = 448 -> s = 1
    q, s = oracle.quant_per_token(row, oracle.FMT_E4M3)
    assert s[0] == 1.0
    assert np.array_equal(q[0, :0x7F], codes)
    assert np.array_equal(q[0, 0x7F:], codes[1:] | 0x80)


def test_zero_row_gets_unit_scale_and_zero_codes():
    row = np.zeros((2, 256), np.float32)
    row[1] = -0.0
    for f in (oracle.FMT_E4M3, oracle.FMT_INT8):
        q, s = oracle.quant_per_token(row, f)
        assert np.all(s == 1.0)
        assert np.all(q[0] == 0)
    q, _ = oracle.quant_per_token(row, oracle.FMT_E4M3)
    assert np.all(q[1] == 0x80)                    # -0 keeps its sign in e4m3


def test_quotient_above_448_saturates_instead_of_nan():
    # find bf16 magnitudes a with fl(a / fl(a / 448)) > 448 in fp32
    a = np.arange(0x3F80, 0x4780, dtype=np.uint32) << 16
    a = a.view(np.float32)
    s = (a / np.float32(448)).astype(np.float32)
    over = a[(a / s).astype(np.float32) > np.float32(448)]
    assert over.size > 0
    row = np.array([[over[0], -over[0], over[0] / 2]], np.float32)
    q, _ = oracle.quant_per_token(row, oracle.FMT_E4M3)
    assert q[0, 0] == 0x7E and q[0, 1] == 0xFE


def test_rejects_non_bf16_input():
    with pytest.raises(ValueError):
        oracle.quant_per_token(np.array([[1.0 + 2 ** -20]], np.float32), oracle.FMT_E4M3)
