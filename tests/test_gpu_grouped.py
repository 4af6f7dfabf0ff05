"""GPU parity of the grouped (mixture-of-experts) GEMM against the oracle.

Each expert's rows must meet the single-product rule of its format (INT8:
bf16 within one ulp of the correctly rounded value; FP8 / Block_FP8: the
normwise and 2^-8 * S elementwise bounds); rows a call must not write keep
their sentinel.  Calls go through the C ABI (qlin_grouped_scaled_mm /
qlin_grouped_block_scaled_mm) via the binding, with the device-resident
offset table.
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

TORCH_DT = {"fp8": torch.float8_e4m3fn, "int8": torch.int8, "block_fp8": torch.float8_e4m3fn}
SENTINEL = -12345          # int16 bit pattern of a bf16 NaN-free sentinel value


def say(*a):
    print("[gpu-grouped]", *a, flush=True)
    sys.stdout.flush()


def moe_case(fmt, sizes, N, K, seed=0):
    """Tokens sorted by expert: rows [sum(sizes), K]; experts' weights [G, N, K]."""
    G = len(sizes)
    rows = int(sum(sizes))
    g = synth.rng(71, seed, N, K)
    x = synth.activations(rows, K, g, outliers=fmt != "int8", outlier_key=(71, 3, K))
    w = [synth.weights(N, K, (71, seed, e, N, K)) for e in range(G)]
    if fmt == "block_fp8":
        qa, sa = synth.quant_groups(x)
        qb, sb = zip(*[synth.quant_blocks(we) for we in w])
    else:
        qa, sa = synth.quant_rows(x, fmt)
        qb, sb = zip(*[synth.quant_rows(we, fmt) for we in w])
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return qa, np.asarray(sa, np.float32), np.stack(qb), np.stack(sb).astype(np.float32), off


def to_dev(fmt, qa, sa, qb, sb, off):
    dt = TORCH_DT[fmt]
    return (torch.from_numpy(np.ascontiguousarray(qa)).cuda().view(dt),
            torch.from_numpy(np.ascontiguousarray(sa)).cuda(),
            torch.from_numpy(np.ascontiguousarray(qb)).cuda().view(dt),
            torch.from_numpy(np.ascontiguousarray(sb)).cuda(),
            torch.from_numpy(off).cuda())


def run(fmt, dev, max_rows, cfg=None):
    a, sa, b, sb, off = dev
    out = torch.full((a.shape[0], b.shape[1]), SENTINEL, dtype=torch.int16,
                     device="cuda").view(torch.bfloat16)
    if fmt == "block_fp8":
        q.grouped_block_scaled_mm(a, sa, b, sb, off, max_rows, out=out, config=cfg)
    else:
        q.grouped_scaled_mm(a, sa, b, sb, off, max_rows, out=out, config=cfg)
    torch.cuda.synchronize()
    return parity.y_bits(out)


def check(fmt, y, qa, sa, qb, sb, off, max_rows, what=""):
    """Per expert: the rows it computes meet the format's rule against the
    single-product oracle; rows past max_rows keep the sentinel."""
    block = fmt == "block_fp8"
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        cut = min(hi, lo + max_rows)
        if cut > lo:
            ref = oracle.scaled_mm(parity.FMT_CODE[fmt], qa[lo:cut], sa[lo:cut], qb[e], sb[e],
                                   block=block)
            parity.check_y(fmt, y[lo:cut], ref.y, ref.ydbl, ref.bound, f"{what} expert {e}")
        assert np.all(y[cut:hi].view(np.int16) == SENTINEL), f"{what} expert {e} rows past max_rows"


# decode-like routing: many experts, 0-6 tokens each; prefill-like: a few
# experts with hundreds of tokens (several tile rows)
DECODE_SIZES = [2, 0, 1, 5, 0, 0, 3, 6, 1, 0, 2, 4]
PREFILL_SIZES = [130, 0, 257, 64, 1]


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_grouped_matches_oracle(fmt, kind):
    sizes = DECODE_SIZES if kind == "decode" else PREFILL_SIZES
    N, K = (384, 1024) if kind == "decode" else (256, 512)
    say(fmt, kind, sizes, N, K)
    qa, sa, qb, sb, off = moe_case(fmt, sizes, N, K, seed=1)
    dev = to_dev(fmt, qa, sa, qb, sb, off)
    max_rows = max(sizes)
    y = run(fmt, dev, max_rows)
    check(fmt, y, qa, sa, qb, sb, off, max_rows, f"{fmt} {kind}")


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_every_instance_grouped(fmt):
    # every built kernel family runs grouped (split_k = 1, grid.z = expert)
    sizes = [3, 0, 17, 40, 1]
    N, K = 256, 1024
    qa, sa, qb, sb, off = moe_case(fmt, sizes, N, K, seed=2)
    dev = to_dev(fmt, qa, sa, qb, sb, off)
    max_rows = max(sizes)
    first = None
    for cfg in q.instances_for(fmt):
        c = cfg.replace(split_k=1, reduce=q.REDUCE_LAST_ARRIVER)
        if q.check_config(fmt, max_rows, N, K, c) != 0:
            continue
        if c.kernel == q.KERNEL_STREAM_TOK:
            # the persistent token-stationary kernel has no grouped form: refused
            with pytest.raises(q.QlinError) as e:
                run(fmt, dev, max_rows, c)
            assert e.value.status == 6, e.value
            continue
        say(fmt, "instance", c)
        y = run(fmt, dev, max_rows, c)
        check(fmt, y, qa, sa, qb, sb, off, max_rows, f"{fmt} {c}")
        if fmt == "int8":
            first = y if first is None else first
            assert np.array_equal(y, first), f"int8 instance disagreement at {c}"


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("max_rows", [1, 2, 3])
def test_few_rows_per_expert_default_kernel(fmt, max_rows):
    # decode routing with at most 3 rows per expert at K >= 2048: the
    # default grouped choice (the GEMV kernel) against the oracle
    sizes = [min(max_rows, s) for s in (1, 0, 3, 2, 1, 0, 3)]
    N, K = 384, 2048
    c = q.select_grouped_config(fmt, max_rows, N, K)
    say(fmt, "few rows", max_rows, c)
    assert c.kernel == q.KERNEL_GEMV
    qa, sa, qb, sb, off = moe_case(fmt, sizes, N, K, seed=6)
    dev = to_dev(fmt, qa, sa, qb, sb, off)
    y = run(fmt, dev, max_rows)
    check(fmt, y, qa, sa, qb, sb, off, max_rows, f"{fmt} few rows {max_rows}")


def test_max_rows_caps_each_group():
    # rows of a group past max_rows are left untouched (documented bound)
    sizes = [5, 9, 0, 12]
    qa, sa, qb, sb, off = moe_case("fp8", sizes, 256, 512, seed=3)
    dev = to_dev("fp8", qa, sa, qb, sb, off)
    y = run("fp8", dev, 4)
    check("fp8", y, qa, sa, qb, sb, off, 4, "cap")


def test_single_group_equals_scaled_mm():
    # one expert over all rows is the ordinary call, bit for bit (same kernel
    # and config, split_k = 1)
    M, N, K = 29, 512, 1024
    qa, sa, qb, sb, off = moe_case("int8", [M], N, K, seed=4)
    dev = to_dev("int8", qa, sa, qb, sb, off)
    c = q.select_config("int8", M, N, K).replace(split_k=1, reduce=q.REDUCE_LAST_ARRIVER)
    y = run("int8", dev, M, c)
    a, sa_d, b, sb_d, _ = dev
    y1 = q.scaled_mm(a, sa_d, b[0], sb_d[0], config=c)
    assert np.array_equal(y, parity.y_bits(y1))


def test_all_groups_empty_and_graph_replay():
    # no tokens routed anywhere writes nothing; a captured grouped call
    # replays with new routing (offsets read on the device at run time)
    sizes = [4, 0, 7]
    N, K = 256, 512
    qa, sa, qb, sb, off = moe_case("fp8", sizes, N, K, seed=5)
    a, sa_d, b, sb_d, off_d = to_dev("fp8", qa, sa, qb, sb, off)
    out = torch.full((a.shape[0], N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    zero = torch.zeros(4, dtype=torch.int32, device="cuda")
    q.grouped_scaled_mm(a, sa_d, b, sb_d, zero, 8, out=out)
    torch.cuda.synchronize()
    assert np.all(parity.y_bits(out).view(np.int16) == SENTINEL)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.grouped_scaled_mm(a, sa_d, b, sb_d, off_d, 8, out=out)
    for routing in ([4, 0, 7], [0, 11, 0], [2, 2, 7]):
        o = np.concatenate([[0], np.cumsum(routing)]).astype(np.int32)
        off_d.copy_(torch.from_numpy(o))
        out.view(torch.int16).fill_(SENTINEL)
        g.replay()
        torch.cuda.synchronize()
        check("fp8", parity.y_bits(out), qa, sa, qb, sb, o, 8, f"replay {routing}")


# ---------------------------------------------------------------------------
# Every grouped entry of the tuned table at its full size: a 128-expert top-8
# layer of the 30B-class mixture-of-experts model, routed by the seeded
# uniform routing at the token count the entry was tuned on, with real
# quantized weights; the library's own selection must be the entry's config.
# Checked at 1500 sampled outputs (plus every expert's first and last row).
# ---------------------------------------------------------------------------
import functools
import os

from tests.test_gpu_full_size import table_entries

GROUPED_ENTRIES = table_entries(grouped=True)
TUNED_BATCHES = (1, 4, 16, 32, 64, 128, 512, 2048)


@functools.lru_cache(maxsize=1)
def moe_weights(fmt, N, K):
    E = synth.MOE_EXPERTS
    qb, sb = [], []
    for e in range(E):
        w = synth.weights(N, K, (72, e, N, K))
        b, s = synth.quant_blocks(w) if fmt == "block_fp8" else synth.quant_rows(w, fmt)
        qb.append(b)
        sb.append(s)
    return np.stack(qb), np.stack(sb).astype(np.float32)


def batch_for(M, K):
    for b in TUNED_BATCHES:
        if int(synth.moe_counts(b, K).max()) == M:
            return b
    raise AssertionError(f"no tuned batch routes at most {M} rows to an expert (K={K})")


@pytest.mark.parametrize("fmt,M,N,K,cfg", GROUPED_ENTRIES,
                         ids=[f"{f}-rows{M}-N{N}-K{K}" for (f, M, N, K, _) in GROUPED_ENTRIES])
def test_grouped_table_entry_full_size(fmt, M, N, K, cfg):
    sel = q.select_grouped_config(fmt, M, N, K)
    assert sel == cfg, f"the library selects {sel}, the table says {cfg}"
    batch = batch_for(M, K)
    counts = synth.moe_counts(batch, K)
    rows = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.activations(rows, K, (73, batch, K), outliers=fmt != "int8", outlier_key=(73, 3, K))
    qa, sa = synth.quant_groups(x) if fmt == "block_fp8" else synth.quant_rows(x, fmt)
    qb, sb = moe_weights(fmt, N, K)
    say("grouped full", fmt, "batch", batch, "max_rows", M, (N, K), cfg)
    y = run(fmt, to_dev(fmt, qa, sa, qb, sb, off), M)
    # sampled positions: every active expert's first and last row, then random rows
    g = np.random.default_rng(5)
    act = [e for e in range(len(counts)) if counts[e] > 0]
    ms = [int(off[e]) for e in act] + [int(off[e + 1]) - 1 for e in act]
    ms += list(g.integers(0, rows, 1500))
    ns = list(g.integers(0, N, len(ms)))
    ms, ns = np.asarray(ms), np.asarray(ns)
    expert = np.searchsorted(off, ms, side="right") - 1
    block = fmt == "block_fp8"
    for e in np.unique(expert):
        sel_e = expert == e
        lo = int(off[e])
        r = oracle.scaled_mm_points(parity.FMT_CODE[fmt], qa[lo:int(off[e + 1])], sa[lo:int(off[e + 1])],
                                    qb[e], sb[e], ms[sel_e] - lo, ns[sel_e], block=block)
        parity.check_y(fmt, y[ms[sel_e], ns[sel_e]], r.y, r.ydbl, r.bound, f"{fmt} expert {e}")
