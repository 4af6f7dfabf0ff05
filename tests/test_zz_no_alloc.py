"""The allocation-free entry point (qlin_scaled_mm_noalloc) against the
entry point it varies (qlin_scaled_mm / qlin_block_scaled_mm with a caller
workspace), through the C ABI.

Same config, same kernels: the outputs must be bit-identical, and both must
meet the oracle's rule (tests/parity.py).  Two calls in a row, the second
smaller, so the second reads a scratch array holding the first call's
partials (and, for the last-arriver reduction, the counters the first call
left re-armed).  Also a capture/replay of the new entry point, and the
error for a config whose workspace exceeds the scratch array.
"""
import sys

import numpy as np
import pytest
import torch

import int8_gemm_linear_amd as q
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def nan_out(M, N):
    return torch.full((M, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def both(case):
    ops = parity.to_device(case)
    ref_out = nan_out(case.M, case.N)
    if case.block:
        q.block_scaled_mm(*ops, out=ref_out)
    else:
        q.scaled_mm(*ops, out=ref_out)
    out = nan_out(case.M, case.N)
    q.scaled_mm_noalloc(*ops, out=out, block=case.block)
    torch.cuda.synchronize()
    return ref_out, out, ops


# (first, second): the second call is smaller.  Each call must use split-K
# (two-pass reduction at tuned table entries, the last-arriver one at untuned
# shapes); candidate shapes per slot, the first whose selection splits is used,
# so retuning the table cannot quietly turn a case into one without scratch.
PAIRS = [
    ((("fp8", 32, 5120, 25600), ("fp8", 128, 4096, 4096)), (("fp8", 24, 5120, 25600), ("fp8", 8, 768, 4096))),
    ((("int8", 32, 5120, 25600), ("int8", 32, 3072, 6144)), (("int8", 16, 1024, 8192),)),
    ((("block_fp8", 32, 5120, 25600), ("block_fp8", 32, 12288, 4096)),
     (("block_fp8", 8, 5120, 25600), ("block_fp8", 8, 1024, 8192))),
    ((("int8", 32, 3072, 6144),), (("int8", 16, 1024, 8192),)),
    ((("fp8", 12, 1536, 2048),), (("fp8", 8, 768, 4096),)),
]


def first_split(options):
    for fmt, M, N, K in options:
        if q.select_config(fmt, M, N, K).split_k > 1:
            return fmt, M, N, K
    raise AssertionError(f"no candidate shape selects split-K: {options}")


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a[0][0]}-{i}" for i, (a, b) in enumerate(PAIRS)])
def test_noalloc_matches_workspace_entry_point(first, second):
    shapes = [first_split(first), first_split(second)]
    assert shapes[1][1] * shapes[1][2] < shapes[0][1] * shapes[0][2], shapes   # the second is smaller
    for fmt, M, N, K in shapes:
        cfg = q.select_config(fmt, M, N, K)
        case = synth.make_case(fmt, M, N, K, root=61)
        say("noalloc", fmt, (M, N, K), cfg)
        ref_out, out, _ = both(case)
        assert np.array_equal(parity.y_bits(out), parity.y_bits(ref_out)), (fmt, M, N, K)
        parity.check_sampled(case, out, npts=1500) if M * N > 64 * 1024 else parity.check_case(case, out)


def test_noalloc_graph_replay():
    fmt, M, N, K = "fp8", 8, 768, 4096            # split 8, last-arriver counters
    case = synth.make_case(fmt, M, N, K, root=62)
    ref_out, _, ops = both(case)
    out = nan_out(M, N)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.scaled_mm_noalloc(*ops, out=out)
    for rep in range(3):
        out.view(torch.int16).fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        say("noalloc replay", rep)
        assert np.array_equal(parity.y_bits(out), parity.y_bits(ref_out)), rep
        # an eager call of another shape between replays uses the same scratch
        other = synth.make_case("int8", 16, 1024, 8192, root=63)
        r2, o2, _ = both(other)
        assert np.array_equal(parity.y_bits(o2), parity.y_bits(r2))


def test_noalloc_too_large_workspace_is_rejected():
    from tests.test_abi import oversize_shape
    fmt, M, N, K = oversize_shape()
    block = fmt == "block_fp8"
    dt = torch.int8 if fmt == "int8" else torch.float8_e4m3fn
    a = torch.zeros((M, K), dtype=torch.uint8, device="cuda").view(dt)
    b = torch.zeros((N, K), dtype=torch.uint8, device="cuda").view(dt)
    sa = torch.ones((M, K // 128) if block else (M,), device="cuda")
    sb = torch.ones((N // 128, K // 128) if block else (N,), device="cuda")
    out = nan_out(M, N)
    with pytest.raises(q.QlinError) as e:
        q.scaled_mm_noalloc(a, sa, b, sb, out=out, block=block)
    assert e.value.status == 5
