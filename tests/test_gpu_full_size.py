"""Full-size parity at every entry of the tuned config table, and past the
decode range the table was tuned on.

Each entry of configs/qlin_mi355x.cfg is one (format, N, K, M) point of the
workloads, run at its full size with the library's own selection (which must
be that entry's config: the launch configuration the benchmark times) and
checked against the oracle at the four corners plus 1500 seeded positions
(whole output when it is small).  Large per-shape config files are hard to
validate exhaustively ("Building a High-Performance and Portable vLLM Linear
Backend with Helion", section "Challenges"); this table is small enough to
run in full.  Token counts 33-128 sit past the 32-token boundary of the
pages' hybrid dispatch (techfeed summary, section on hybrid dispatch), where
this library still serves the call itself through the nearest table entry
or its built-in default.
"""
import os
import sys

import pytest
import torch

import int8_gemm_linear_amd as q
import synth
from tests import parity

pytestmark = pytest.mark.gpu

TABLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "int8_gemm_linear_amd", "configs", "qlin_mi355x.cfg")


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def table_entries(grouped=False):
    """(fmt, M, N, K, Config) of every ordinary (or every grouped) table line."""
    out = []
    for line in open(TABLE):
        line = line.split("#", 1)[0].split()
        if not line or (line[0] == "grouped") != grouped:
            continue
        if grouped:
            line = line[1:]
        fmt = line[0]
        N, K, M = (int(v) for v in line[1:4])
        cfg = q.Config(*(int(v) for v in line[4:14]))
        out.append((fmt, M, N, K, cfg))
    # weights are generated once per (fmt, N, K) and cached across M
    out.sort(key=lambda e: (e[0], e[2], e[3], e[1]))
    return out


ENTRIES = table_entries()

# One shape per model class and format, at token counts past the tuned decode
# grid {1, 2, 4, 8, 16, 24, 32} and below the prefill points.
BOUNDARY_M = (33, 48, 64, 96, 128)
BOUNDARY = [("int8", M, 4096, 2048) for M in BOUNDARY_M] + \
    [(f, M, 6144, 4096) for f in ("fp8", "block_fp8") for M in BOUNDARY_M] + \
    [(f, M, 5120, 8192) for f in ("int8", "fp8", "block_fp8") for M in BOUNDARY_M]


def make(fmt, M, N, K):
    if (fmt, M, N, K) == ("fp8", 16, 512, 1024):
        return synth.make_case_seed0(fmt, M, N, K)
    return synth.make_case(fmt, M, N, K)


def run_and_check(case):
    a, sa, b, sb = parity.to_device(case)
    out = torch.full((case.M, case.N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if case.block:
        q.block_scaled_mm(a, sa, b, sb, out=out)
    else:
        q.scaled_mm(a, sa, b, sb, out=out)
    torch.cuda.synchronize()
    if case.M * case.N <= 64 * 1024:
        return parity.check_case(case, out)
    return parity.check_sampled(case, out, npts=1500)


def test_table_has_every_workload_point():
    pts = {p for w in ("fp8_small", "int8_1p7b_decode", "fp8_8b", "block_fp8_8b", "all_32b")
           for p in synth.workload(w)}
    assert {(f, M, N, K) for (f, M, N, K, _) in ENTRIES} == pts
    assert len(ENTRIES) + len(table_entries(grouped=True)) == q.config_table_size()


@pytest.mark.parametrize("fmt,M,N,K,cfg", ENTRIES,
                         ids=[f"{f}-M{M}-N{N}-K{K}" for (f, M, N, K, _) in ENTRIES])
def test_table_entry_full_size(fmt, M, N, K, cfg):
    sel = q.select_config(fmt, M, N, K)
    assert sel == cfg, f"the library selects {sel}, the table says {cfg}"
    say("full", fmt, (M, N, K), cfg)
    stats = run_and_check(make(fmt, M, N, K))
    say("  ok", stats)


@pytest.mark.parametrize("fmt,M,N,K", BOUNDARY,
                         ids=[f"{f}-M{M}-N{N}-K{K}" for (f, M, N, K) in BOUNDARY])
def test_past_the_decode_range_full_size(fmt, M, N, K):
    say("boundary", fmt, (M, N, K), q.select_config(fmt, M, N, K))
    stats = run_and_check(make(fmt, M, N, K))
    say("  ok", stats)


# The persistent token-stationary kernel at the 32B-class decode shapes, at
# its own full-size grid (several weight tiles per workgroup), every instance
# that takes the shape with the fewest splits its token area allows.
TOK_POINTS = [(f, M, N, K) for f in ("int8", "fp8") for M in (16, 32)
              for (N, K) in ((51200, 5120), (5120, 8192))]


@pytest.mark.parametrize("fmt,M,N,K", TOK_POINTS, ids=[f"{f}-M{M}-N{N}-K{K}" for (f, M, N, K) in TOK_POINTS])
def test_token_stationary_full_size(fmt, M, N, K):
    case = make(fmt, M, N, K)
    a, sa, b, sb = parity.to_device(case)
    n = 0
    for c in q.instances_for(fmt):
        if c.kernel != q.KERNEL_STREAM_TOK or c.tile_m < M:
            continue
        def cfg(split):
            return c.replace(split_k=split,
                             reduce=q.REDUCE_TWO_PASS if split > 1 else q.REDUCE_LAST_ARRIVER)
        split = 1
        while q.check_config(fmt, M, N, K, cfg(split)) != 0:
            split *= 2
            assert split <= 256
        cc = cfg(split)
        say("token stationary full", fmt, (M, N, K), cc)
        out = torch.full((M, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        q.scaled_mm(a, sa, b, sb, out=out, config=cc)
        torch.cuda.synchronize()
        say("  ok", parity.check_sampled(case, out, npts=1500))
        n += 1
    assert n > 0
