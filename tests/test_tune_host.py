"""Host-side checks of the tuner's candidate set (CPU only): which kernel
families and splits it offers per token count, and that every candidate is
a configuration the library accepts for the point."""
import int8_gemm_linear_amd as q
from int8_gemm_linear_amd.tune import candidates


def kinds(cands):
    return {c.kernel for c in cands}


def test_every_candidate_is_accepted():
    for fmt, M, N, K in (("int8", 1, 2048, 2048), ("fp8", 24, 4096, 4096),
                         ("block_fp8", 2, 5120, 8192), ("fp8", 2048, 5120, 8192)):
        cands = candidates(fmt, M, N, K)
        assert cands, (fmt, M, N, K)
        for c in cands:
            assert q.check_config(fmt, M, N, K, c) == 0, (fmt, M, N, K, c)


def test_token_count_decides_the_families():
    one = candidates("int8", 1, 2048, 2048)
    assert q.KERNEL_GEMV in kinds(one) and q.KERNEL_STREAM_LDS in kinds(one)
    assert q.KERNEL_TILE not in kinds(one)                   # tiles start at 16 tokens
    # GEMV only for token counts its tile covers in one workgroup column
    for M in (1, 2, 4, 8, 16):
        for c in candidates("int8", M, 2048, 2048):
            if c.kernel == q.KERNEL_GEMV:
                assert M <= c.tile_m, (M, c)
    big = candidates("fp8", 2048, 5120, 8192)
    assert kinds(big) == {q.KERNEL_TILE}                      # stream kernels stop at 4 token tiles


def test_gemv_candidates_take_no_split():
    for fmt in ("int8", "fp8", "block_fp8"):
        g = [c for c in candidates(fmt, 1, 4096, 4096) if c.kernel == q.KERNEL_GEMV]
        assert g, fmt
        assert all(c.split_k == 1 for c in g), fmt


def test_splits_are_powers_of_two_within_the_k_steps():
    K = 2048
    for c in candidates("int8", 8, 2048, K):
        s = c.split_k
        assert s & (s - 1) == 0 and 1 <= s <= 256
        assert s <= K // 128


def test_wide_row_ring_offered_at_16_to_32_tokens():
    # The wide-row LDS ring (tile_k = 256: 128 or 256 weight rows per
    # workgroup, each wave owning whole 16-row blocks) is Swap-AB only, for
    # every format, and offered from 16 tokens (its 16- and 32-token tiles)
    # with and without split-K; K must be whole 256-byte chunks.
    for fmt in ("int8", "fp8", "block_fp8"):
        wide = [c for c in q.instances_for(fmt) if c.kernel == q.KERNEL_STREAM_LDS and c.tile_k == 256]
        assert {(c.tile_m, c.tile_n) for c in wide} == {(16, 128), (32, 128), (16, 256), (32, 256)}, fmt
        assert all(c.variant == q.SWAP_AB for c in wide), fmt
        assert {c.waves_n for c in wide} == {1, 2}, fmt          # tile and spread placement
        for M in (16, 24, 32):
            cw = [c for c in candidates(fmt, M, 51200, 5120)
                  if c.kernel == q.KERNEL_STREAM_LDS and c.tile_k == 256]
            assert cw and {c.split_k for c in cw} >= {1, 2, 4}, (fmt, M)
        assert not [c for c in candidates(fmt, 4, 51200, 5120)
                    if c.kernel == q.KERNEL_STREAM_LDS and c.tile_k == 256], fmt
        c = wide[0]
        assert q.check_config(fmt, 32, 51200, 5120, c) == 0
        assert q.check_config(fmt, 32, 51200, 5120 + 128, c) != 0   # K % 256 != 0


def test_table_picks_the_wide_ring_on_the_widest_decode_shape():
    # the tuned table's choice at 16-32 tokens on (K, N) = (5120, 51200),
    # all three formats, is the wide-row ring with spread placement
    for fmt in ("int8", "fp8", "block_fp8"):
        for M in (16, 24, 32):
            c = q.select_config(fmt, M, 51200, 5120)
            assert (c.kernel, c.tile_k, c.tile_n, c.waves_n) == (q.KERNEL_STREAM_LDS, 256, 256, 2), (fmt, M, c)
