"""Lifetime of the binding's split-K workspaces under HIP graph capture.

A captured graph replays with the workspace address it was captured with.
These tests grow the eager workspace after a capture (which once freed the
buffer the graph still used), grow a workspace inside a capture, and replay
with unrelated allocations and eager work in between; every replay must
still match the oracle.  Rules as everywhere: INT8 within one bf16 ulp of the
oracle (tests/parity.py).
"""
import functools
import sys

import pytest
import torch

import int8_gemm_linear_amd as q
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def case_and_ref(M, N, K):
    c = synth.make_case("int8", M, N, K, root=41)
    return c, parity.oracle_full(c)


def split_cfg(M, N, K, split, reduce):
    # the register stream kernel at 16 weight rows x 32 tokens, split over K
    cfg = q.Config(kernel=q.KERNEL_STREAM, variant=q.SWAP_AB, tile_m=32, tile_n=16, tile_k=512,
                   waves_n=1, waves_k=4, stages=2, split_k=split, reduce=reduce)
    assert q.check_config("int8", M, N, K, cfg) == 0, cfg
    return cfg


def run(case, cfg, out):
    a, sa, b, sb = parity.to_device(case)
    return q.scaled_mm(a, sa, b, sb, out=out, config=cfg), (a, sa, b, sb)


def nan_out(M, N):
    return torch.full((M, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


@pytest.mark.parametrize("reduce", [q.REDUCE_LAST_ARRIVER, q.REDUCE_TWO_PASS])
def test_eager_growth_after_capture_keeps_graph_valid(reduce):
    small = (32, 1024, 2048)            # split 4: 0.5 MiB of partials
    large = (64, 4096, 2048)            # split 8: 8 MiB of partials (grows the buffer)
    cs, rs = case_and_ref(*small)
    cl, rl = case_and_ref(*large)
    cfg_s = split_cfg(*small, 4, reduce)
    cfg_l = split_cfg(*large, 8, reduce)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        say("eager small", small, cfg_s)
        y0 = nan_out(small[0], small[1])
        run(cs, cfg_s, y0)
        s.synchronize()
        parity.check_case(cs, y0, rs, what="eager small")
        ops = parity.to_device(cs)
        yg = nan_out(small[0], small[1])
        g = torch.cuda.CUDAGraph()
        say("capture small")
        with torch.cuda.graph(g, stream=s):
            q.scaled_mm(*ops, out=yg, config=cfg_s)
        say("eager large (grows the eager workspace)")
        yl = nan_out(large[0], large[1])
        run(cl, cfg_l, yl)
        s.synchronize()
        parity.check_case(cl, yl, rl, what="eager large")
    # fill freed memory, if any, with junk before every replay
    junk = [torch.full((1 << 20,), 0x7F7F7F7F, dtype=torch.int32, device="cuda") for _ in range(16)]
    for rep in range(3):
        yg.view(torch.int16).fill_(-1)
        with torch.cuda.stream(s):
            g.replay()
            s.synchronize()
        say("replay", rep)
        parity.check_case(cs, yg, rs, what=f"replay {rep}")
        # eager work on the same stream between replays
        with torch.cuda.stream(s):
            run(cl, cfg_l, yl)
            s.synchronize()
        parity.check_case(cl, yl, rl, what=f"eager large after replay {rep}")
    del junk, g


def test_growth_inside_one_capture():
    # the second call of the capture needs a larger workspace than the first
    small = (32, 1024, 2048)
    large = (64, 4096, 2048)
    cs, rs = case_and_ref(*small)
    cl, rl = case_and_ref(*large)
    cfg_s = split_cfg(*small, 4, q.REDUCE_LAST_ARRIVER)
    cfg_l = split_cfg(*large, 8, q.REDUCE_LAST_ARRIVER)
    ops_s, ops_l = parity.to_device(cs), parity.to_device(cl)
    ys, yl = nan_out(small[0], small[1]), nan_out(large[0], large[1])
    g = torch.cuda.CUDAGraph()
    say("capture small + large")
    with torch.cuda.graph(g):
        q.scaled_mm(*ops_s, out=ys, config=cfg_s)
        q.scaled_mm(*ops_l, out=yl, config=cfg_l)
        q.scaled_mm(*ops_s, out=ys, config=cfg_s)
    for rep in range(3):
        ys.view(torch.int16).fill_(-1)
        yl.view(torch.int16).fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        say("replay", rep)
        parity.check_case(cs, ys, rs, what=f"small, replay {rep}")
        parity.check_case(cl, yl, rl, what=f"large, replay {rep}")


def test_streams_get_distinct_workspaces():
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    dev = torch.device("cuda", torch.cuda.current_device())
    w1 = q.workspace_for(1 << 20, dev, s1)
    w2 = q.workspace_for(1 << 20, dev, s2)
    torch.cuda.synchronize()
    assert w1.data_ptr() != w2.data_ptr()
    assert q.workspace_for(1 << 10, dev, s1).data_ptr() == w1.data_ptr()
