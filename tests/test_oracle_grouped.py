"""Pins of the oracle's grouped (mixture-of-experts) product (CPU only).

Grouped GEMM, the MoE target named in the ai-radar commentary "Helion in
vLLM: il tuning dei GEMM diventa ricerca…", section "Oltre Hopper:
Blackwell, AMD, TPU e il perimetro del fork": many experts, each a small
scaled_mm over its own tokens and weights.  The oracle composes the pinned
single-product oracle over the groups; these tests pin the composition
against invariants that do not go through it group by group.
"""
import numpy as np
import pytest

import oracle
import synth


def case(fmt, rows, N, K, G, seed):
    g = synth.rng(61, seed)
    x = synth.activations(rows, K, g)
    w = np.stack([synth.weights(N, K, (61, seed, e)) for e in range(G)])
    if fmt == "block_fp8":
        qa, sa = synth.quant_groups(x)
        qb, sb = zip(*[synth.quant_blocks(w[e]) for e in range(G)])
    else:
        qa, sa = synth.quant_rows(x, fmt)
        qb, sb = zip(*[synth.quant_rows(w[e], fmt) for e in range(G)])
    return qa, sa, np.stack(qb), np.stack(sb)


FMT = {"fp8": oracle.FMT_E4M3, "int8": oracle.FMT_INT8, "block_fp8": oracle.FMT_E4M3}


@pytest.mark.parametrize("fmt", ["fp8", "int8", "block_fp8"])
def test_same_weights_for_every_group_is_one_product(fmt):
    # all experts share one weight matrix: the grouped result is the single
    # product over all rows (catches a row offset or group stride mistake)
    rows, N, K, G = 23, 256, 256, 5
    qa, sa, qb, sb = case(fmt, rows, N, K, 1, 1)
    qbG = np.repeat(qb, G, axis=0)
    sbG = np.repeat(sb, G, axis=0)
    off = [0, 4, 4, 11, 20, 23]
    y = oracle.grouped_scaled_mm(FMT[fmt], off, qa, sa, qbG, sbG, block=fmt == "block_fp8")
    ref = oracle.scaled_mm(FMT[fmt], qa, sa, qb[0], sb[0], block=fmt == "block_fp8").y
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("fmt", ["fp8", "block_fp8"])
def test_permuting_experts_permutes_rows(fmt):
    # experts reordered together with their token blocks: the output rows move
    # with them (catches weights paired with the wrong group)
    rows, N, K, G = 19, 128, 256, 4
    qa, sa, qb, sb = case(fmt, rows, N, K, G, 2)
    off = np.array([0, 3, 10, 10, 19])
    y = oracle.grouped_scaled_mm(FMT[fmt], off, qa, sa, qb, sb, block=fmt == "block_fp8")
    perm = [2, 0, 3, 1]
    blocks = [np.arange(off[g], off[g + 1]) for g in range(G)]
    order = np.concatenate([blocks[g] for g in perm])
    off2 = np.concatenate([[0], np.cumsum([len(blocks[g]) for g in perm])])
    y2 = oracle.grouped_scaled_mm(FMT[fmt], off2, qa[order], sa[order], qb[perm], sb[perm],
                                  block=fmt == "block_fp8")
    assert np.array_equal(y2, y[order])


def test_distinct_weights_differ_per_group_and_max_rows_caps():
    rows, N, K, G = 12, 128, 128, 3
    qa, sa, qb, sb = case("int8", rows, N, K, G, 3)
    off = [0, 5, 5, 12]
    y = oracle.grouped_scaled_mm(oracle.FMT_INT8, off, qa, sa, qb, sb)
    # group 0 with expert 2's weights gives a different result (weights matter)
    y_wrong = oracle.scaled_mm(oracle.FMT_INT8, qa[:5], sa[:5], qb[2], sb[2]).y
    assert not np.array_equal(y[:5], y_wrong)
    # max_rows = 2: only the first two rows of each group are computed
    init = np.full((rows, N), 0x1234, np.uint16)
    yc = oracle.grouped_scaled_mm(oracle.FMT_INT8, off, qa, sa, qb, sb, max_rows=2, Y=init)
    for lo, hi in ((0, 5), (5, 12)):
        assert np.array_equal(yc[lo:lo + 2], y[lo:lo + 2])
        assert np.all(yc[lo + 2:hi] == 0x1234)
