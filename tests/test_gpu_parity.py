"""GPU parity of the HIP path against the CPU oracle (MI355X).

Every call goes through the C ABI of libqlinear.so via the binding.
Rules (tests/parity.py): INT8 accumulators bit-exact and outputs within one
bf16 ulp; FP8 / Block_FP8 normwise <= 1e-2 and |err| <= 2^-8 * S elementwise.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import int8_gemm_linear_amd as q
import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def small_case(fmt, M, N, K, root=21):
    return synth.make_case(fmt, M, N, K, root=root)


@functools.lru_cache(maxsize=None)
def small_ref(fmt, M, N, K, root=21):
    return parity.oracle_full(small_case(fmt, M, N, K, root))


def call(case, dev, cfg=None, out=None):
    a, sa, b, sb = dev
    if out is None:
        # NaN-filled, so an output the kernels fail to write cannot pass
        out = torch.full((case.M, case.N), -1, dtype=torch.int16, device=a.device).view(torch.bfloat16)
    if case.block:
        return q.block_scaled_mm(a, sa, b, sb, out=out, config=cfg)
    return q.scaled_mm(a, sa, b, sb, out=out, config=cfg)


# Ragged shapes spanning several tiles: M not a multiple of 16/32, N not a
# multiple of the tile (token/channel formats), K several 128-byte steps.
SHAPE = {"fp8": (37, 300, 1024), "int8": (37, 300, 1024), "block_fp8": (37, 384, 1024)}


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_every_instance_matches_oracle(fmt):
    M, N, K = SHAPE[fmt]
    case = small_case(fmt, M, N, K)
    ref = small_ref(fmt, M, N, K)
    dev = parity.to_device(case)
    first = None
    for cfg in q.instances_for(fmt):
        splits = ((1, 1), (2, q.REDUCE_LAST_ARRIVER), (4, q.REDUCE_TWO_PASS))
        if cfg.kernel == q.KERNEL_GEMV:
            splits = splits[:1]               # a GEMV wave covers a row's whole K
        if cfg.kernel == q.KERNEL_STREAM_TOK:
            splits = ((1, 1), (2, q.REDUCE_TWO_PASS), (4, q.REDUCE_TWO_PASS))   # two-pass only
        for split, red in splits:
            c = cfg.replace(split_k=split, reduce=red)
            assert q.check_config(fmt, M, N, K, c) == 0, c
            say(fmt, (M, N, K), c)
            y = call(case, dev, c)
            torch.cuda.synchronize()
            parity.check_case(case, y, ref, what=f"{fmt} {c}")
            if fmt == "int8":
                yb = parity.y_bits(y)
                if first is None:
                    first = yb
                # W8A8_INT8: every variant / split gives the same bits (exact int32 sums)
                assert np.array_equal(yb, first), f"int8 variant disagreement at {c}"


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_tile_instances_one_and_two_token_tiles(fmt):
    # The tile kernel has two copy forms chosen at launch: one token tile
    # (M <= tile_m: weight copies non-temporal) and several token tiles.
    # Every tile instance runs both: M = tile_m - 3 and M = tile_m + 3.
    N, K = (384, 1024)
    for c in q.instances_for(fmt):
        if c.kernel != q.KERNEL_TILE:
            continue
        for M in (c.tile_m - 3, c.tile_m + 3):
            case = small_case(fmt, M, N, K, root=26)
            ref = small_ref(fmt, M, N, K, root=26)
            say("tile copy forms", fmt, M, c)
            y = call(case, parity.to_device(case), c)
            torch.cuda.synchronize()
            parity.check_case(case, y, ref, what=f"{fmt} M={M} {c}")


def test_int8_accumulators_bit_exact():
    M, N, K = SHAPE["int8"]
    case = small_case("int8", M, N, K)
    ref = small_ref("int8", M, N, K)
    a, _, b, _ = parity.to_device(case)
    for cfg in q.instances_for("int8"):
        for split, red in ((1, 1), (4, q.REDUCE_LAST_ARRIVER), (8, q.REDUCE_TWO_PASS)):
            c = cfg.replace(split_k=split, reduce=red)
            if q.check_config("int8", M, N, K, c) != 0:
                continue                      # e.g. more splits than the kernel's K units
            say("int8 acc", c)
            acc = q.int8_accumulate(a, b, config=c,
                                    out=torch.full((M, N), -2 ** 31, dtype=torch.int32, device="cuda"))
            torch.cuda.synchronize()
            assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref.acc), c


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_every_token_count_1_to_32(fmt):
    N, K = (256, 1024)
    for M in range(1, 33):
        case = small_case(fmt, M, N, K, root=22)
        say(fmt, "M", M)
        y = call(case, parity.to_device(case))
        torch.cuda.synchronize()
        parity.check_case(case, y)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_k_not_multiple_of_128(fmt):
    # K % 16 == 0 is all the ABI asks; the stream kernel masks the last step.
    for M, N, K in ((5, 96, 16), (17, 130, 1040), (40, 64, 208)):
        case = small_case(fmt, M, N, K, root=23)
        say(fmt, (M, N, K))
        y = call(case, parity.to_device(case))
        torch.cuda.synchronize()
        parity.check_case(case, y)


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_gemv_ragged_k_and_rows(fmt):
    # every GEMV instance at 1-2 tokens on K that ends inside a 1 KB row
    # segment (and, token/channel formats, inside a 128-byte step), N not a
    # multiple of the rows per workgroup: pieces past K are zeroed, rows past
    # N are never stored
    shapes = ((1, 77, 1040), (2, 130, 2064), (1, 33, 6160)) if fmt != "block_fp8" else \
             ((1, 256, 1152), (2, 384, 2176), (1, 128, 6272))
    gemv = [c for c in q.instances_for(fmt) if c.kernel == q.KERNEL_GEMV]
    assert gemv
    for M, N, K in shapes:
        case = small_case(fmt, M, N, K, root=29)
        dev = parity.to_device(case)
        ref = parity.oracle_full(case)
        for c in gemv:
            if q.check_config(fmt, M, N, K, c) != 0:
                continue
            say(fmt, "gemv", (M, N, K), c)
            y = call(case, dev, c)
            torch.cuda.synchronize()
            parity.check_case(case, y, ref, what=f"{fmt} {c} {(M, N, K)}")


def test_split_k_sweep():
    M, N, K = 24, 512, 4096
    for fmt in ("int8", "fp8", "block_fp8"):
        case = small_case(fmt, M, N, K, root=24)
        ref = parity.oracle_full(case)
        dev = parity.to_device(case)
        base = q.select_config(fmt, M, N, K)
        for split in (1, 2, 4, 8, 16, 32):
            for red in (q.REDUCE_TWO_PASS, q.REDUCE_LAST_ARRIVER):
                c = base.replace(split_k=split, reduce=red)
                if q.check_config(fmt, M, N, K, c) != 0:
                    continue
                say(fmt, c)
                y = call(case, dev, c)
                torch.cuda.synchronize()
                parity.check_case(case, y, ref, what=f"{fmt} {c}")


def test_fp8_run_to_run_reproducible():
    M, N, K = 32, 1024, 4096
    for fmt in ("fp8", "block_fp8"):
        case = small_case(fmt, M, N, K, root=25)
        dev = parity.to_device(case)
        base = q.select_config(fmt, M, N, K)
        for c in (base.replace(split_k=8, reduce=q.REDUCE_LAST_ARRIVER),
                  base.replace(split_k=8, reduce=q.REDUCE_TWO_PASS)):
            say("repro", fmt, c)
            ys = [parity.y_bits(call(case, dev, c)) for _ in range(10)]
            for y in ys[1:]:
                assert np.array_equal(y, ys[0])


def test_exhaustive_code_pairs_on_gpu():
    # One non-zero per row (k = 0): every product of two codes, scales 1.
    for fmt in ("fp8", "int8"):
        codes = np.arange(256, dtype=np.uint8)
        if fmt == "fp8":
            codes = codes[(codes & 0x7F) != 0x7F]
        K = 16
        A = np.zeros((codes.size, K), np.uint8)
        A[:, 0] = codes
        ones = np.ones(codes.size, np.float32)
        case = synth.Case(fmt, codes.size, codes.size, K, A, ones, A.copy(), ones.copy())
        say("pairs", fmt)
        y = call(case, parity.to_device(case))
        torch.cuda.synchronize()
        ref = parity.oracle_full(case)
        got = parity.y_bits(y)
        zero = (ref.y & 0x7FFF) == 0
        assert np.array_equal(got[~zero], ref.y[~zero])
        assert ((got[zero] & 0x7FFF) == 0).all()


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_identity_weights_on_gpu(fmt):
    K = 512
    case = small_case(fmt, 9, K, K, root=26)
    one = 1 if fmt == "int8" else 0x38
    B = np.zeros((K, K), np.uint8)
    B[np.arange(K), np.arange(K)] = one
    sB = np.ones((K // 128, K // 128), np.float32) if fmt == "block_fp8" else np.ones(K, np.float32)
    c2 = synth.Case(fmt, 9, K, K, case.A, case.sA, B, sB)
    say("identity", fmt)
    y = call(c2, parity.to_device(c2))
    torch.cuda.synchronize()
    parity.check_case(c2, y)


def test_output_stride_and_guard_bands():
    M, N, K = 20, 200, 1024
    for fmt in ("int8", "fp8"):
        case = small_case(fmt, M, N, K, root=27)
        dev = parity.to_device(case)
        big = torch.full((M + 2, N + 40), 0x7777, dtype=torch.int16, device="cuda")
        out = big.view(torch.bfloat16)[1:M + 1, 8:8 + N]
        for c in (q.select_config(fmt, M, N, K),
                  q.select_config(fmt, M, N, K).replace(split_k=4, reduce=q.REDUCE_TWO_PASS)):
            say("guard", fmt, c)
            y = call(case, dev, c, out=out)
            torch.cuda.synchronize()
            parity.check_case(case, y.contiguous())
            g = big.cpu().numpy().copy()
            g[1:M + 1, 8:8 + N] = 0x7777
            assert (g == 0x7777).all(), "write outside the output view"


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_gemv_strided_operands_and_guard_bands(fmt):
    # every GEMV instance with lda > K, ldb > K and an output view inside a
    # guarded buffer: results as the oracle's, nothing written outside
    M, N, K = 2, 256, 2048
    case = small_case(fmt, M, N, K, root=31)
    a, sa, b, sb = parity.to_device(case)
    ap = torch.zeros((M, K + 48), dtype=torch.uint8, device="cuda")
    bp = torch.zeros((N, K + 32), dtype=torch.uint8, device="cuda")
    ap[:, :K] = a.view(torch.uint8)
    bp[:, :K] = b.view(torch.uint8)
    a2, b2 = ap.view(a.dtype)[:, :K], bp.view(b.dtype)[:, :K]
    ref = parity.oracle_full(case)
    for c in [c for c in q.instances_for(fmt) if c.kernel == q.KERNEL_GEMV]:
        if q.check_config(fmt, M, N, K, c) != 0:
            continue
        big = torch.full((M + 2, N + 40), 0x7777, dtype=torch.int16, device="cuda")
        out = big.view(torch.bfloat16)[1:M + 1, 8:8 + N]
        say("gemv strides", fmt, c)
        f = q.block_scaled_mm if case.block else q.scaled_mm
        f(a2, sa, b2, sb, out=out, config=c)
        torch.cuda.synchronize()
        parity.check_case(case, out.contiguous(), ref, what=f"{fmt} {c}")
        g = big.cpu().numpy().copy()
        g[1:M + 1, 8:8 + N] = 0x7777
        assert (g == 0x7777).all(), f"write outside the output view: {c}"


def test_hip_graph_capture_and_replay():
    M, N, K = 16, 2048, 2048
    for fmt in ("int8", "fp8", "block_fp8"):
        case = small_case(fmt, M, N, K, root=28)
        dev = parity.to_device(case)
        cfg = q.select_config(fmt, M, N, K).replace(split_k=8, reduce=q.REDUCE_LAST_ARRIVER)
        eager = call(case, dev, cfg).clone()
        torch.cuda.synchronize()
        out = torch.empty_like(eager)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(case, dev, cfg, out=out)           # warm-up, allocates the workspace
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(case, dev, cfg, out=out)
        for r in range(3):
            say("graph replay", fmt, r)
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), (fmt, r)
            _ = torch.ones(1024, device="cuda").sum().item()   # eager work between replays
        parity.check_case(case, out)


def test_empty_inputs():
    for fmt in ("int8", "fp8"):
        dt = torch.int8 if fmt == "int8" else torch.float8_e4m3fn
        a = torch.zeros((0, 128), dtype=torch.uint8, device="cuda").view(dt)
        b = torch.zeros((64, 128), dtype=torch.uint8, device="cuda").view(dt)
        y = q.scaled_mm(a, torch.ones(0, device="cuda"), b, torch.ones(64, device="cuda"))
        assert y.shape == (0, 64)


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_spread_row_placement(fmt):
    # LDS-ring kernel with rows shared evenly over a grid sized to the CUs
    # (waves_n = 2): workgroups start at any multiple of 8 rows, hold several
    # 8-row units, and (Block_FP8) straddle 128-row weight blocks.  Every tile
    # width, both orientations, with and without split-K.
    for M, N, K in ((32, 5120, 1024), (16, 2944, 2048), (5, 1280, 512)):
        case = small_case(fmt, M, N, K, root=24)
        ref = small_ref(fmt, M, N, K, root=24)
        dev = parity.to_device(case)
        first = None
        cfgs = {}
        for c in q.instances_for(fmt):
            if c.kernel == q.KERNEL_STREAM_LDS and c.waves_n == 2 and M <= c.tile_m <= 2 * max(M, 8):
                cfgs.setdefault((c.tile_n, c.variant), c)
        assert cfgs
        for c in cfgs.values():
            for split, red in ((1, 1), (2, q.REDUCE_LAST_ARRIVER), (2, q.REDUCE_TWO_PASS)):
                cc = c.replace(split_k=split, reduce=red)
                if q.check_config(fmt, M, N, K, cc) != 0:
                    continue
                say("spread", fmt, (M, N, K), cc)
                y = call(case, dev, cc)
                torch.cuda.synchronize()
                parity.check_case(case, y, ref, what=f"{fmt} {cc}")
                if fmt == "int8":
                    yb = parity.y_bits(y)
                    first = yb if first is None else first
                    assert np.array_equal(yb, first), f"int8 disagreement at {cc}"


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_deep_rings_long_k(fmt):
    # Every LDS-ring instance with three or more stages on a K long enough to
    # cycle its ring several times (K = 12288: 12-24 chunks), both placements,
    # with and without split-K.
    M, N, K = 20, (384 if fmt == "block_fp8" else 300), 12288
    case = small_case(fmt, M, N, K, root=25)
    ref = small_ref(fmt, M, N, K, root=25)
    dev = parity.to_device(case)
    first = None
    for c in q.instances_for(fmt):
        if c.kernel != q.KERNEL_STREAM_LDS or c.stages < 3 or -(-M // c.tile_m) > 4:
            continue
        for split, red in ((1, 1), (2, q.REDUCE_TWO_PASS)):
            cc = c.replace(split_k=split, reduce=red)
            if q.check_config(fmt, M, N, K, cc) != 0:
                continue
            say("deep ring", fmt, cc)
            y = call(case, dev, cc)
            torch.cuda.synchronize()
            parity.check_case(case, y, ref, what=f"{fmt} {cc}")
            if fmt == "int8":
                yb = parity.y_bits(y)
                first = yb if first is None else first
                assert np.array_equal(yb, first), f"int8 disagreement at {cc}"


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_token_stationary_kernel(fmt):
    # Persistent kernel with the token rows stationary in LDS (kernel kind 4):
    # every instance on a one-split K (the token area at 64 KB), on a K that
    # needs two splits for 32-token tiles (the area full for 16-token ones),
    # and with 97 tokens (four token tiles, the last ragged) over 32 splits,
    # which leaves 2-4 workgroups per (token tile, split): each holds up to
    # four weight tiles of 16 * waves rows, the last one partial.
    N = 1000
    first = {}
    for M, K, split in ((32, 2048, 1), (13, 5120, 2), (97, 8192, 32)):
        case = small_case(fmt, M, N, K, root=28)
        ref = small_ref(fmt, M, N, K, root=28)
        dev = parity.to_device(case)
        n = 0
        for c in q.instances_for(fmt):
            if c.kernel != q.KERNEL_STREAM_TOK:
                continue
            for s in (split, 2 * split):
                cc = c.replace(split_k=s, reduce=q.REDUCE_TWO_PASS if s > 1 else q.REDUCE_LAST_ARRIVER)
                if q.check_config(fmt, M, N, K, cc) != 0:
                    continue
                say("token stationary", fmt, (M, N, K), cc)
                y = call(case, dev, cc)
                torch.cuda.synchronize()
                parity.check_case(case, y, ref, what=f"{fmt} {cc}")
                n += 1
                if fmt == "int8":
                    yb = parity.y_bits(y)
                    first.setdefault((M, K), yb)
                    assert np.array_equal(yb, first[(M, K)]), f"int8 disagreement at {cc}"
        assert n >= 6, n


@pytest.mark.parametrize("fmt", ["int8", "fp8", "block_fp8"])
def test_wide_row_kernel_at_its_placement(fmt):
    # The wide-row LDS ring (tile_k = 256) as the table uses it on N = 51200:
    # spread placement gives 256 workgroups of 200 rows each, starting at
    # multiples of 8 that are not multiples of 128, so a workgroup's rows
    # span up to three 128-row weight blocks (Block_FP8 scales).  Short K
    # keeps the oracle fast while every output element is compared; 16, 24
    # and 32 tokens, with and without split-K.
    N, K = 51200, 1024
    cfgs = [c for c in q.instances_for(fmt)
            if c.kernel == q.KERNEL_STREAM_LDS and c.tile_k == 256 and c.waves_n == 2]
    assert {c.tile_n for c in cfgs} == {128, 256}, cfgs
    first = {}
    for M in (16, 24, 32):
        case = small_case(fmt, M, N, K, root=29)
        ref = small_ref(fmt, M, N, K, root=29)
        dev = parity.to_device(case)
        for c in cfgs:
            if c.tile_m < M and -(-M // c.tile_m) > 2:
                continue
            for split, red in ((1, 1), (2, q.REDUCE_TWO_PASS), (4, q.REDUCE_LAST_ARRIVER)):
                cc = c.replace(split_k=split, reduce=red)
                assert q.check_config(fmt, M, N, K, cc) == 0, cc
                say("wide rows", fmt, (M, N, K), cc)
                y = call(case, dev, cc)
                torch.cuda.synchronize()
                parity.check_case(case, y, ref, what=f"{fmt} {cc}")
                if fmt == "int8":
                    yb = parity.y_bits(y)
                    first.setdefault(M, yb)
                    assert np.array_equal(yb, first[M]), f"int8 disagreement at {cc}"
