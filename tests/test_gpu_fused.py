"""GPU parity of the fused producers (RMS norm / SiLU-and-mul + dynamic
quantizer) against the CPU oracle (MI355X).

The oracle composes its pinned producer (the real-number value rounded once
to bf16, evaluated in double) with its pinned quantizer.  Codes and scales
are integers / fp32 values decided from that bf16 activation, so the bar is
bit-exact: every code byte, every scale bit pattern and every residual
output equal the oracle's.  The only arithmetic that may differ between the
two sides is the order of the double-precision sum of squares, which moves
the value by far less than a bf16 rounding interval.  Calls go through the C
ABI via the binding.
"""
import sys

import numpy as np
import pytest
import torch

import int8_gemm_linear_amd as q
import oracle
import synth

pytestmark = pytest.mark.gpu

TORCH_DT = {"fp8": torch.float8_e4m3fn, "int8": torch.int8}
ORC_DT = {"fp8": oracle.FMT_E4M3, "int8": oracle.FMT_INT8}
EPS = 1e-6


def say(*a):
    print("[gpu-fused]", *a, flush=True)
    sys.stdout.flush()


def act(M, K, root=41, scale=1.0, outliers=True):
    x = synth.activations(M, K, (root, 2, M, K), outliers=outliers, outlier_key=(root, 3, K))
    return synth.bf16_round(x * np.float32(scale))


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(torch.bfloat16)


def codes(t):
    return t.view(torch.uint8).cpu().numpy()


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def same_scales(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


def run_rms(x, w, fmt, block, residual=None, eps=EPS):
    xd, wd = dev(x), dev(w)
    rd = None if residual is None else dev(residual)
    if block:
        qd, sd = q.rms_norm_per_block_quant(xd, wd, eps, residual=rd)
    else:
        qd, sd = q.rms_norm_dynamic_per_token_quant(xd, wd, eps, TORCH_DT[fmt], residual=rd)
    torch.cuda.synchronize()
    return codes(qd), sd.cpu().numpy(), None if rd is None else bits(rd)


@pytest.mark.parametrize("fmt,block", [("fp8", False), ("int8", False), ("fp8", True)])
@pytest.mark.parametrize("M,K", [(1, 128), (3, 2048), (33, 4096), (5, 5120), (300, 2048),
                                 (2, 40960)])
@pytest.mark.parametrize("with_residual", [False, True])
def test_rms_norm_quant_bit_exact(fmt, block, M, K, with_residual):
    say("rms", fmt, "block" if block else "token", M, K, "residual" if with_residual else "")
    x = act(M, K)
    w = synth.norm_weight(K, (41, 4, K))
    r = act(M, K, root=43, scale=4.0) if with_residual else None
    qd, sd, hd = run_rms(x, w, fmt, block, r)
    qr, sr, hr = oracle.rms_norm_quant(x, w, EPS, ORC_DT[fmt], 128 if block else 0, residual=r)
    if with_residual:
        assert np.array_equal(hd, hr)
    assert same_scales(sd, sr)
    assert np.array_equal(qd, qr)


@pytest.mark.parametrize("fmt,block", [("fp8", False), ("int8", False), ("fp8", True)])
# wave counts 1 (K <= 4096; K = 4096 fills every register slot), 2 (6144)
# and 4 (12288 up, past the register window from 16384)
@pytest.mark.parametrize("M,K", [(1, 128), (7, 6144), (33, 12288), (2, 25600), (3, 40960),
                                 (64, 2048), (32, 4096)])
def test_silu_and_mul_quant_bit_exact(fmt, block, M, K):
    say("silu", fmt, "block" if block else "token", M, K)
    x = act(M, 2 * K, scale=2.0)
    xd = dev(x)
    if block:
        qd, sd = q.silu_and_mul_per_block_quant(xd)
    else:
        qd, sd = q.silu_and_mul_dynamic_per_token_quant(xd, TORCH_DT[fmt])
    torch.cuda.synchronize()
    qr, sr = oracle.silu_and_mul_quant(x, ORC_DT[fmt], 128 if block else 0)
    assert same_scales(sd.cpu().numpy(), sr)
    assert np.array_equal(codes(qd), qr)


@pytest.mark.parametrize("fmt,block", [("fp8", False), ("int8", False), ("fp8", True)])
def test_special_rows(fmt, block):
    # zero row (norm 0 / sqrt(eps) = 0: scale 1, codes 0), values near the
    # bf16 maximum and in the bf16 subnormal range (the sums of squares
    # leave fp32's range; double keeps them), a single non-zero value,
    # SiLU at large |gate| (e^-g overflows / underflows), zero up
    K = 256
    rows = np.zeros((6, K), np.float32)
    rows[1, :] = 3.0e38 * np.where(np.arange(K) % 2, 1.0, -1.0)
    rows[2, :] = 2.0e-39 * (1 + np.arange(K) % 7)
    rows[3, 17] = -5.0
    rows[4, :] = np.linspace(-1000, 1000, K)
    rows[5, :] = np.linspace(-3, 3, K)
    rows = synth.bf16_round(rows)
    w = synth.norm_weight(K, (41, 5, K))
    say("special rms", fmt, block)
    qd, sd, _ = run_rms(rows, w, fmt, block)
    qr, sr, _ = oracle.rms_norm_quant(rows, w, EPS, ORC_DT[fmt], 128 if block else 0)
    assert same_scales(sd, sr)
    assert np.array_equal(qd, qr)
    say("special silu", fmt, block)
    # gate: the rows above; up: 0 (row 0), 0.5 (rows 1-3: no bf16 overflow at
    # a gate of 3e38), a ramp (rows 4-5)
    up = np.zeros((6, K), np.float32)
    up[1:4] = 0.5
    up[4:] = np.linspace(-2, 2, K)
    x = np.concatenate([rows, synth.bf16_round(up)], axis=1)
    xd = dev(x)
    if block:
        qd2, sd2 = q.silu_and_mul_per_block_quant(xd)
    else:
        qd2, sd2 = q.silu_and_mul_dynamic_per_token_quant(xd, TORCH_DT[fmt])
    torch.cuda.synchronize()
    qr2, sr2 = oracle.silu_and_mul_quant(x, ORC_DT[fmt], 128 if block else 0)
    assert same_scales(sd2.cpu().numpy(), sr2)
    assert np.array_equal(codes(qd2), qr2)


def test_strided_rows_and_guard_bytes():
    # ldx > K, ldr > K and ldq > K: bytes outside each row's K untouched
    M, K, ldx, ldq = 9, 1024, 1040, 1056
    say("strided", M, K)
    x = act(M, ldx)
    r = act(M, ldx, root=44)
    w = synth.norm_weight(K, (41, 6, K))
    xd, rd, wd = dev(x), dev(r), dev(w)
    qbuf = torch.full((M, ldq), 0x5A, dtype=torch.uint8, device="cuda")
    qv = qbuf.view(torch.float8_e4m3fn)[:, :K]
    qd, sd = q.rms_norm_dynamic_per_token_quant(xd[:, :K], wd, EPS, torch.float8_e4m3fn,
                                                residual=rd[:, :K], out=qv)
    torch.cuda.synchronize()
    qr, sr, hr = oracle.rms_norm_quant(x[:, :K], w, EPS, oracle.FMT_E4M3,
                                       residual=r[:, :K])
    qb = qbuf.cpu().numpy()
    assert np.array_equal(qb[:, :K], qr)
    assert np.all(qb[:, K:] == 0x5A)
    assert same_scales(sd.cpu().numpy(), sr)
    rb = bits(rd)
    assert np.array_equal(rb[:, :K], hr)
    assert np.array_equal(rb[:, K:], oracle._bf16_bits(r[:, K:]))   # untouched past K
    # SiLU-and-mul with padded rows: x [M, ldx2] holding gate | up in the first 2K
    ldx2 = 2 * K + 64
    x2 = act(M, ldx2, root=45)
    xd2 = dev(x2)
    qbuf.fill_(0x5A)
    q.silu_and_mul_per_block_quant(xd2[:, :2 * K], out=qv)
    torch.cuda.synchronize()
    qr2, _ = oracle.silu_and_mul_quant(x2[:, :2 * K], group=128)
    qb = qbuf.cpu().numpy()
    assert np.array_equal(qb[:, :K], qr2)
    assert np.all(qb[:, K:] == 0x5A)


def test_empty_rows():
    for fn in (lambda x, w: q.rms_norm_dynamic_per_token_quant(x, w),
               lambda x, w: q.rms_norm_per_block_quant(x, w),
               lambda x, w: q.silu_and_mul_dynamic_per_token_quant(torch.cat([x, x], 1)),
               lambda x, w: q.silu_and_mul_per_block_quant(torch.cat([x, x], 1))):
        x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
        w = torch.ones(256, dtype=torch.bfloat16, device="cuda")
        c, s = fn(x, w)
        assert c.shape[0] == 0 and s.shape[0] == 0


@pytest.mark.parametrize("kind", ["rms", "silu"])
def test_full_size_sampled_rows(kind):
    # prefill size of the 32B-class model (hidden 5120, intermediate 25600),
    # M = 2048, in the launch configuration the benchmark times; the oracle
    # checks a sample of rows (the producers are row-independent)
    M, K = 2048, 5120 if kind == "rms" else 25600
    say("full", kind, M, K)
    g = synth.rng(41, 7)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 1], g.choice(M, 12, replace=False)]))
    if kind == "rms":
        x = act(M, K)
        w = synth.norm_weight(K, (41, 8, K))
        qd, sd, _ = run_rms(x, w, "fp8", False)
        qr, sr, _ = oracle.rms_norm_quant(x[rows], w, EPS, oracle.FMT_E4M3)
    else:
        x = act(M, 2 * K, scale=2.0)
        xd = dev(x)
        qd, sd = q.silu_and_mul_per_block_quant(xd)
        torch.cuda.synchronize()
        qd, sd = codes(qd), sd.cpu().numpy()
        qr, sr = oracle.silu_and_mul_quant(x[rows], group=128)
    assert same_scales(sd[rows], sr)
    assert np.array_equal(qd[rows], qr)


def test_fused_equals_unfused_library_path():
    # the fused kernel returns what the library's own quantizer returns on the
    # oracle's bf16 producer output
    M, K = 17, 4096
    x = act(M, K)
    w = synth.norm_weight(K, (41, 9, K))
    y, _ = oracle.rms_norm(x, w, EPS)
    yd = torch.from_numpy(y.view(np.int16)).to("cuda").view(torch.bfloat16)
    qu, su = q.quant_per_token(yd, torch.int8)
    qf, sf, _ = run_rms(x, w, "int8", False)
    assert np.array_equal(codes(qu), qf)
    assert same_scales(su.cpu().numpy(), sf)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("K", [6144, 6160, 25600])
def test_silu_rows_spread_over_workgroups(fmt, K):
    # At a few tokens a per-token SiLU-and-mul row is spread over several
    # workgroups, each of which finds the row maximum itself (its own exact
    # values, then the exact value of every other value whose bound reaches
    # them).  Rows built so the maximum sits where that search must find it:
    # an all-zero row (every bound is a candidate), a maximum through the
    # double path (gate > 64) in the last workgroup's slice, a maximum from a
    # negative gate with a large up value, the maximum value twice in two
    # slices, a maximum in the first slice, and a random row.  K = 6160 makes
    # the last slice two pieces long.
    rng = np.random.default_rng(61)
    M = 6
    g = synth.bf16_round(rng.normal(0.0, 0.01, (M, K)).astype(np.float32))
    u = synth.bf16_round(rng.normal(0.0, 0.01, (M, K)).astype(np.float32))
    g[0] = 0.0
    u[0] = 0.0
    g[1, K - 3], u[1, K - 3] = 100.0, 3.0
    g[2, K // 2 + 5], u[2, K // 2 + 5] = -1.28125, 1000.0
    g[3, 11], u[3, 11] = 2.5, -7.0
    g[3, K - 40], u[3, K - 40] = 2.5, 7.0
    g[4, 3], u[4, 3] = 5.0, 5.0
    g[5] = synth.bf16_round(rng.normal(0.0, 1.0, K).astype(np.float32))
    u[5] = synth.bf16_round(rng.normal(0.0, 1.0, K).astype(np.float32))
    x = np.concatenate([g, u], axis=1)
    say("silu spread", fmt, M, K)
    qd, sd = q.silu_and_mul_dynamic_per_token_quant(dev(x), TORCH_DT[fmt])
    torch.cuda.synchronize()
    qr, sr = oracle.silu_and_mul_quant(x, ORC_DT[fmt], 0)
    assert same_scales(sd.cpu().numpy(), sr)
    assert np.array_equal(codes(qd), qr)
