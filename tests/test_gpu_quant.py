"""GPU parity of the activation quantizers against the CPU oracle (MI355X).

Codes are integers decided in fp32, so the bar is bit-exact: every code byte
and every scale's bit pattern equal the oracle's.  Calls go through the C ABI
(qlin_quant_per_token / qlin_quant_per_group128) via the binding.
"""
import sys

import numpy as np
import pytest
import torch

import int8_gemm_linear_amd as q
import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

TORCH_DT = {"fp8": torch.float8_e4m3fn, "int8": torch.int8}
ORC_DT = {"fp8": oracle.FMT_E4M3, "int8": oracle.FMT_INT8}


def say(*a):
    print("[gpu-quant]", *a, flush=True)
    sys.stdout.flush()


def act(M, K, root=31, outliers=True):
    return synth.activations(M, K, (root, 2, M, K), outliers=outliers, outlier_key=(root, 3, K))


def to_dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(torch.bfloat16)


def codes(t):
    return t.view(torch.uint8).cpu().numpy()


def same_scales(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("M,K", [(1, 16), (1, 2048), (7, 1040), (33, 4096), (5, 5120),
                                 (3, 25600), (2, 40960), (300, 2048)])
def test_per_token_bit_exact(fmt, M, K):
    say("per_token", fmt, M, K)
    x = act(M, K)
    qd, sd = q.quant_per_token(to_dev_bf16(x), TORCH_DT[fmt])
    torch.cuda.synchronize()
    qr, sr = oracle.quant_per_token(x, ORC_DT[fmt])
    assert same_scales(sd.cpu().numpy(), sr)
    assert np.array_equal(codes(qd), qr)


@pytest.mark.parametrize("M,K", [(1, 128), (5, 1024), (33, 5120), (300, 2048), (2, 25600)])
def test_per_group_bit_exact(M, K):
    say("per_group", M, K)
    x = act(M, K)
    qd, sd = q.quant_per_group128(to_dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr = oracle.quant_per_group(x, 128)
    assert same_scales(sd.cpu().numpy(), sr)
    assert np.array_equal(codes(qd), qr)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_special_rows(fmt):
    # zero row, negative-zero row, halves (int8 ties), the e4m3 grid itself,
    # a single large value, subnormal-range values
    K = 256
    rows = np.zeros((6, K), np.float32)
    rows[1] = -0.0
    rows[2, :8] = [127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 126.5, -127.0]
    grid = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    rows[3, :127] = grid
    rows[3, 127:254] = -grid
    rows[4, 17] = -3.0e4
    rows[4, 18] = 1.0
    rows[5, :] = np.float32(2.0 ** -12)
    rows[5, 3] = np.float32(1.0)
    x = synth.bf16_round(rows)
    say("special", fmt)
    qd, sd = q.quant_per_token(to_dev_bf16(x), TORCH_DT[fmt])
    torch.cuda.synchronize()
    qr, sr = oracle.quant_per_token(x, ORC_DT[fmt])
    assert same_scales(sd.cpu().numpy(), sr)
    assert np.array_equal(codes(qd), qr)
    if fmt == "fp8":
        qg, sg = q.quant_per_group128(to_dev_bf16(x))
        torch.cuda.synchronize()
        qgr, sgr = oracle.quant_per_group(x, 128)
        assert same_scales(sg.cpu().numpy(), sgr)
        assert np.array_equal(codes(qg), qgr)


def test_strided_rows_leave_guard_bytes():
    M, K, ldx, ldq = 9, 1024, 1024 + 64, 1024 + 48
    x = act(M, K)
    xs = torch.zeros((M, ldx), dtype=torch.bfloat16, device="cuda")
    xs[:, :K] = to_dev_bf16(x)
    qs = torch.full((M, ldq), 0x5A, dtype=torch.uint8, device="cuda")
    sd = torch.empty((M,), dtype=torch.float32, device="cuda")
    say("strided per_token")
    q.quant_per_token(xs[:, :K], torch.float8_e4m3fn, out=qs[:, :K].view(torch.float8_e4m3fn), scale=sd)
    torch.cuda.synchronize()
    qr, sr = oracle.quant_per_token(x, oracle.FMT_E4M3)
    host = qs.cpu().numpy()
    assert np.array_equal(host[:, :K], qr)
    assert np.all(host[:, K:] == 0x5A)
    assert same_scales(sd.cpu().numpy(), sr)


def test_empty_is_noop():
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    qd, sd = q.quant_per_token(x)
    qg, sg = q.quant_per_group128(x)
    torch.cuda.synchronize()
    assert qd.shape == (0, 1024) and sd.shape == (0,) and sg.shape == (0, 8)


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_full_size_sampled_rows(fmt):
    # prefill activation of the 32B-class (K=25600) linear at M=2048, in the
    # launch configuration of the library; the oracle checks sampled rows
    M, K = 2048, 25600
    x = act(M, K, root=7)
    xd = to_dev_bf16(x)
    say("full", fmt, M, K)
    if fmt == "block_fp8":
        qd, sd = q.quant_per_group128(xd)
    else:
        qd, sd = q.quant_per_token(xd, TORCH_DT[fmt])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 511, 1024, 1500, 2046, 2047])
    xr = x[rows]
    if fmt == "block_fp8":
        qr, sr = oracle.quant_per_group(xr, 128)
    else:
        qr, sr = oracle.quant_per_token(xr, ORC_DT[fmt])
    qh = codes(qd)[rows]
    sh = sd.cpu().numpy()[rows]
    assert same_scales(sh, sr)
    assert np.array_equal(qh, qr)


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_quantize_then_gemm_matches_oracle(fmt):
    # the producer feeding the GEMM: quantize on the GPU, multiply on the GPU,
    # compare with the oracle GEMM on the oracle's own codes
    M, N, K = 24, 512, 2048
    x = act(M, K, root=3)
    case = synth.make_case(fmt, M, N, K, root=3)
    say("quant+gemm", fmt)
    xd = to_dev_bf16(x)
    b = torch.from_numpy(np.ascontiguousarray(case.B)).to("cuda").view(TORCH_DT.get(fmt, torch.float8_e4m3fn))
    sb = torch.from_numpy(np.ascontiguousarray(case.sB)).to("cuda")
    if fmt == "block_fp8":
        qa, sa = q.quant_per_group128(xd)
        y = q.block_scaled_mm(qa, sa, b, sb)
        qr, sr = oracle.quant_per_group(x, 128)
    else:
        qa, sa = q.quant_per_token(xd, TORCH_DT[fmt])
        y = q.scaled_mm(qa, sa, b, sb)
        qr, sr = oracle.quant_per_token(x, ORC_DT[fmt])
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(parity.FMT_CODE[fmt], qr, sr, case.B, case.sB, block=fmt == "block_fp8")
    parity.check_y(fmt, parity.y_bits(y), ref.y, ref.ydbl, ref.bound, "quant+gemm")
