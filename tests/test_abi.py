"""The C ABI on the host (no GPU needed): exported symbols, argument
validation, config selection and the config-table parser.  Every call here
fails validation or is a pure host query, so no kernel is launched."""
import ctypes
import os
import re

import pytest

import int8_gemm_linear_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "qlinear.h")

ST = {"ok": 0, "null": 1, "shape": 2, "stride": 3, "align": 4, "ws": 5, "cfg": 6, "file": 7,
      "hip": 8, "arg": 9}
A16 = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
B16 = 0x20000
Y16 = 0x30000
S4 = 0x40000


def declared_functions():
    text = open(HDR).read()
    return sorted(set(re.findall(r"\b(qlin_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    lib = q.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert q.abi_version() == 1


def smm(dt=q.INT8, M=16, N=256, K=1024, A=A16, lda=None, sA=S4, B=B16, ldb=None, sB=S4,
        Y=Y16, ldy=None, ws=None, wsb=0, cfg=None):
    lib = q.lib()
    args = [dt, M, N, K, A, K if lda is None else lda, sA, B, K if ldb is None else ldb, sB, Y,
            N if ldy is None else ldy, ws, wsb, None]
    if cfg is None:
        return lib.qlin_scaled_mm(*args)
    c = cfg._c()
    return lib.qlin_scaled_mm_cfg(*args, ctypes.byref(c))


def bmm(M=16, N=256, K=1024, **kw):
    lib = q.lib()
    return lib.qlin_block_scaled_mm(M, N, K, A16, K, S4, B16, K, S4, Y16, N, None, 0, None)


def test_shape_errors():
    assert smm(M=-1) == ST["shape"]
    assert smm(N=-3) == ST["shape"]
    assert smm(K=0) == ST["shape"]
    assert smm(K=24) == ST["shape"]                     # K % 16 != 0
    assert smm(dt=q.INT8, K=131072) == ST["shape"]      # int32 accumulator could overflow
    assert bmm(N=200) == ST["shape"]                    # block: N % 128
    assert bmm(K=1040) == ST["shape"]                   # block: K % 128


def test_empty_problems_are_noops():
    assert smm(M=0, A=None, sA=None, B=None, sB=None, Y=None) == ST["ok"]
    assert smm(N=0, A=None, sA=None, B=None, sB=None, Y=None) == ST["ok"]


def test_null_pointer_errors():
    assert smm(A=None) == ST["null"]
    assert smm(B=None) == ST["null"]
    assert smm(sA=None) == ST["null"]
    assert smm(sB=None) == ST["null"]
    assert smm(Y=None) == ST["null"]


def test_stride_and_alignment_errors():
    assert smm(lda=512) == ST["stride"]
    assert smm(lda=1032) == ST["stride"]                # not a multiple of 16
    assert smm(ldb=1000) == ST["stride"]
    assert smm(ldy=100) == ST["stride"]
    assert smm(A=A16 + 1) == ST["align"]
    assert smm(B=B16 + 8) == ST["align"]
    assert smm(Y=Y16 + 2) == ST["align"]
    assert smm(sA=S4 + 2) == ST["align"]


def test_bad_enum():
    assert smm(dt=7) == ST["arg"]


def some_stream_cfg(fmt="int8"):
    for c in q.instances_for(fmt):
        if c.kernel == q.KERNEL_STREAM:
            return c
    raise AssertionError("no stream instance")


def test_gemv_takes_no_split():
    g = [c for c in q.instances_for("int8") if c.kernel == q.KERNEL_GEMV]
    assert g, "no GEMV instance"
    assert q.check_config("int8", 1, 2048, 2048, g[0]) == 0
    assert q.check_config("int8", 1, 2048, 2048, g[0].replace(split_k=2)) == ST["cfg"]
    assert smm(cfg=g[0].replace(split_k=2)) == ST["cfg"]               # rejected before any launch
    blk = [c for c in q.instances_for("block_fp8") if c.kernel == q.KERNEL_GEMV]
    assert blk and all(c.tile_m <= 2 and c.stages == 2 for c in blk)


def test_explicit_config_errors():
    c = some_stream_cfg()
    assert smm(cfg=c.replace(split_k=3)) == ST["cfg"]
    assert smm(cfg=c.replace(split_k=512)) == ST["cfg"]
    assert smm(K=256, cfg=c.replace(split_k=4)) == ST["cfg"]        # more splits than 128-byte steps
    assert smm(cfg=c.replace(reduce=5)) == ST["cfg"]
    assert smm(cfg=c.replace(tile_n=48)) == ST["cfg"]               # no such instance
    # last-arriver needs one counter per output tile inside the 128 KiB region
    many = c.replace(split_k=2, reduce=q.REDUCE_LAST_ARRIVER)
    assert smm(M=16 * 2048, N=c.tile_n * 32, cfg=many, ws=0x50000, wsb=1 << 40) == ST["cfg"]
    tile = [x for x in q.instances_for("int8") if x.kernel == q.KERNEL_TILE][0]
    assert smm(M=256, K=1040, cfg=tile) == ST["cfg"]                # tile kernel needs K % 128 == 0
    # block-scaled configs exist only as built for that format
    blk = q.instances_for("block_fp8")
    std_tile_fp8 = [x for x in q.instances_for("fp8") if x.kernel == q.KERNEL_TILE and x.variant == 0][0]
    assert std_tile_fp8 not in blk


def test_workspace_errors_and_size():
    c = some_stream_cfg().replace(split_k=4, reduce=q.REDUCE_LAST_ARRIVER)
    need = q.workspace_size("int8", 16, 256, 1024, c)
    rnd = lambda v: (v + 255) // 256 * 256
    counters = 128 * 1024                   # fixed counter region, then the partials
    assert need == counters + rnd(4 * 16 * 256 * 4)
    assert q.workspace_size("int8", 16, 256, 1024, c.replace(reduce=q.REDUCE_TWO_PASS)) == need
    assert q.workspace_size("int8", 16, 256, 1024, c.replace(split_k=1)) == 0
    assert smm(cfg=c) == ST["ws"]
    assert smm(cfg=c, ws=0x50000, wsb=need - 1) == ST["ws"]
    assert smm(cfg=c, ws=0x50008, wsb=need) == ST["align"]


def test_every_instance_is_accepted_for_a_compatible_shape():
    for cfg, mask in q.kernel_instances():
        for fmt, bit in (("fp8", 1), ("int8", 2), ("block_fp8", 4)):
            if mask & bit:
                assert q.check_config(fmt, 64, 256, 1024, cfg) == 0, (fmt, cfg)


def test_default_selection_covers_all_workload_shapes():
    import synth
    for name in synth.WORKLOADS:
        for fmt, M, N, K in synth.workload(name):
            c = q.select_config(fmt, M, N, K)
            assert q.check_config(fmt, M, N, K, c) == 0, (fmt, M, N, K, c)
            assert 1 <= c.split_k <= 256 and c.split_k & (c.split_k - 1) == 0


def test_default_configs_are_valid_for_untuned_shapes():
    # shapes outside the tuned table get the built-in choice: always a valid
    # config, the tile kernel for prefill token counts
    for fmt in ("fp8", "int8", "block_fp8"):
        for M in (1, 17, 65, 128, 512, 1024, 2048, 4096):
            for N in (128, 1152, 4224, 51328):
                for K in (128, 1152, 4224, 25728):
                    c = q.select_config(fmt, M, N, K)
                    assert q.check_config(fmt, M, N, K, c) == 0, (fmt, M, N, K, c)
                    if M > 64:
                        assert c.kernel == q.KERNEL_TILE, (fmt, M, N, K, c)
                        assert c.split_k == 1 or K // 128 >= 8 * c.split_k


def test_config_table_file(tmp_path):
    c = some_stream_cfg("fp8")
    line = lambda M, split: (f"fp8 4096 2048 {M} {c.kernel} {c.variant} {c.tile_m} {c.tile_n} "
                             f"{c.tile_k} {c.waves_n} {c.waves_k} {c.stages} {split} 1\n")
    p = tmp_path / "t.cfg"
    p.write_text("# comment\n\n" + line(8, 2) + line(32, 4) + "  # trailing\n")
    base = q.config_table_size()
    q.load_config_table(str(p))
    try:
        assert q.config_table_size() == 2
        assert q.select_config("fp8", 1, 4096, 2048).split_k == 2     # smallest tuned M >= 1
        assert q.select_config("fp8", 8, 4096, 2048).split_k == 2
        assert q.select_config("fp8", 9, 4096, 2048).split_k == 4
        assert q.select_config("fp8", 64, 4096, 2048).split_k == 4    # beyond: the largest M
        # far beyond a decode-only table (M > 64 and > 2x the largest M): the
        # built-in prefill default, not a decode config
        assert q.select_config("fp8", 500, 4096, 2048).kernel == q.KERNEL_TILE
        bad = tmp_path / "bad.cfg"
        bad.write_text("fp8 4096 2048 8 0 1\n")
        with pytest.raises(q.QlinError) as e:
            q.load_config_table(str(bad))
        assert e.value.status == ST["file"]
        assert q.config_table_size() == 2                            # previous table kept
        with pytest.raises(q.QlinError):
            q.load_config_table(str(tmp_path / "missing.cfg"))
        bad.write_text("fp16 4096 2048 8 0 1 16 64 256 2 2 2 1 1\n")
        with pytest.raises(q.QlinError):
            q.load_config_table(str(bad))
    finally:
        q.load_config_table(None)
    assert q.config_table_size() == base


def test_status_strings():
    lib = q.lib()
    for s in range(10):
        assert lib.qlin_status_string(s)


def test_compiled_in_table_entries_are_valid():
    """Every entry of the shipped table names a built instance valid for its own shape."""
    path = os.path.join(ROOT, "int8_gemm_linear_amd", "configs", "qlin_mi355x.cfg")
    n = 0
    for ln in open(path):
        f = ln.split("#")[0].split()
        if not f:
            continue
        grouped = f[0] == "grouped"
        f = f[1:] if grouped else f
        fmt, N, K, M = f[0], int(f[1]), int(f[2]), int(f[3])
        c = q.Config(*[int(x) for x in f[4:14]])
        assert q.check_config(fmt, M, N, K, c) == 0, ln
        if grouped:
            assert c.split_k == 1, ln
            assert q.select_grouped_config(fmt, M, N, K) == c, ln
        else:
            assert q.select_config(fmt, M, N, K) == c, ln
        n += 1
    assert n == q.config_table_size()


def qtok(dt=q.E4M3, M=4, K=1024, X=A16, ldx=None, Q=B16, ldq=None, S=S4):
    return q.lib().qlin_quant_per_token(dt, M, K, X, K if ldx is None else ldx, Q,
                                        K if ldq is None else ldq, S, None)


def qgrp(M=4, K=1024, X=A16, ldx=None, Q=B16, ldq=None, S=S4):
    return q.lib().qlin_quant_per_group128(M, K, X, K if ldx is None else ldx, Q,
                                           K if ldq is None else ldq, S, None)


def test_quant_validation_errors():
    assert qtok(dt=5) == ST["arg"]
    assert qtok(M=-1) == ST["shape"]
    assert qtok(K=0) == ST["shape"]
    assert qtok(K=24) == ST["shape"]
    assert qgrp(K=1040) == ST["shape"]                  # groups need K % 128
    assert qtok(M=0, X=None, Q=None, S=None) == ST["ok"]
    assert qgrp(M=0, X=None, Q=None, S=None) == ST["ok"]
    assert qtok(X=None) == ST["null"]
    assert qtok(S=None) == ST["null"]
    assert qgrp(Q=None) == ST["null"]
    assert qtok(ldx=1000) == ST["stride"]               # ldx < K
    assert qtok(ldx=1028) == ST["stride"]               # ldx % 8
    assert qtok(ldq=1032) == ST["stride"]               # ldq % 16
    assert qtok(X=A16 + 8) == ST["align"]
    assert qgrp(Q=B16 + 4) == ST["align"]
    assert qtok(S=S4 + 2) == ST["align"]


def frms(dt=q.E4M3, M=4, K=1024, X=A16, ldx=None, R=None, ldr=0, W=B16, eps=1e-6, Q=B16,
         ldq=None, S=S4, block=False):
    lib = q.lib()
    if block:
        return lib.qlin_rms_norm_per_block_quant(M, K, X, K if ldx is None else ldx, R, ldr, W,
                                                 eps, Q, K if ldq is None else ldq, S, None)
    return lib.qlin_rms_norm_dynamic_per_token_quant(dt, M, K, X, K if ldx is None else ldx, R, ldr,
                                                     W, eps, Q, K if ldq is None else ldq, S, None)


def fsilu(dt=q.E4M3, M=4, K=1024, X=A16, ldx=None, Q=B16, ldq=None, S=S4, block=False):
    lib = q.lib()
    ldx = 2 * K if ldx is None else ldx
    if block:
        return lib.qlin_silu_and_mul_per_block_quant(M, K, X, ldx, Q, K if ldq is None else ldq,
                                                     S, None)
    return lib.qlin_silu_and_mul_dynamic_per_token_quant(dt, M, K, X, ldx, Q,
                                                         K if ldq is None else ldq, S, None)


def test_fused_producer_validation_errors():
    # argument checks return before any launch (no GPU needed)
    assert frms(dt=7) == ST["arg"]
    assert fsilu(dt=7) == ST["arg"]
    assert frms(K=24) == ST["shape"]
    assert frms(K=1040, block=True) == ST["shape"]          # 1x128 groups need K % 128
    assert fsilu(K=1040, block=True) == ST["shape"]
    assert frms(M=-1) == ST["shape"]
    assert fsilu(K=1 << 20) == ST["shape"]                  # 2K columns past the limit
    assert frms(M=0, X=None, W=None, Q=None, S=None) == ST["ok"]
    assert fsilu(M=0, X=None, Q=None, S=None) == ST["ok"]
    assert frms(W=None) == ST["null"]
    assert frms(X=None) == ST["null"]
    assert fsilu(S=None, block=True) == ST["null"]
    assert frms(ldx=1000) == ST["stride"]
    assert fsilu(ldx=2040) == ST["stride"]                  # rows of 2K values
    assert frms(R=A16, ldr=1000) == ST["stride"]
    assert frms(R=A16, ldr=1028) == ST["stride"]
    assert frms(ldq=1032) == ST["stride"]
    assert frms(W=B16 + 8) == ST["align"]
    assert frms(R=A16 + 8, ldr=1024) == ST["align"]
    assert fsilu(X=A16 + 8) == ST["align"]
    assert frms(eps=-1.0) == ST["arg"]
    assert frms(eps=0.0) == ST["arg"]
    assert frms(eps=float("inf")) == ST["arg"]
    assert frms(eps=float("nan")) == ST["arg"]


def grp(dt=q.E4M3, G=4, off=S4, max_rows=8, N=256, K=1024, A=A16, lda=None, sa=S4, B=B16,
        ldb=None, bstride=None, sb=S4, sbstride=256, Y=B16, ldy=None, block=False, cfg=None):
    lib = q.lib()
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    bstride = N * ldb if bstride is None else bstride
    ldy = N if ldy is None else ldy
    if block:
        return lib.qlin_grouped_block_scaled_mm(G, off, max_rows, N, K, A, lda, sa, B, ldb, bstride,
                                                sb, sbstride, Y, ldy, None, cfg)
    return lib.qlin_grouped_scaled_mm(dt, G, off, max_rows, N, K, A, lda, sa, B, ldb, bstride, sb,
                                      sbstride, Y, ldy, None, cfg)


def test_grouped_validation_errors():
    # argument checks return before any launch (no GPU needed)
    assert grp(dt=9) == ST["arg"]
    assert grp(G=-1) == ST["shape"]
    assert grp(G=0, off=None) == ST["ok"]                  # no groups: no-op
    assert grp(max_rows=0, off=None) == ST["ok"]           # no rows: no-op
    assert grp(G=65536) == ST["shape"]
    assert grp(K=24) == ST["shape"]
    assert grp(N=200, block=True) == ST["shape"]           # block needs N % 128
    assert grp(off=None) == ST["null"]
    assert grp(off=S4 + 2) == ST["align"]
    assert grp(bstride=8) == ST["stride"]                  # group stride % 16
    assert grp(bstride=-16) == ST["stride"]
    assert grp(sbstride=-1) == ST["stride"]
    assert grp(lda=1000) == ST["stride"]
    assert grp(A=A16 + 8) == ST["align"]
    c = q.select_config("fp8", 8, 256, 1024).replace(split_k=2, reduce=0)
    assert grp(cfg=ctypes.byref(c._c())) == ST["cfg"]      # grid.z is the group


def test_grouped_default_config_is_valid_and_unsplit():
    for fmt in ("fp8", "int8", "block_fp8"):
        for mr in (1, 3, 4, 16, 17, 64, 65, 300):
            for (N, K) in ((1536, 2048), (2048, 768), (256, 1024)):
                c = q.select_grouped_config(fmt, mr, N, K)
                assert c.split_k == 1, (fmt, mr, c)
                assert q.check_config(fmt, mr, N, K, c) == 0, (fmt, mr, N, K, c)
                # shapes without grouped table entries follow the built-in
                # rule: GEMV for at most 3 rows per expert at K >= 2048
                # (token/channel formats), the LDS-ring kernel below that K
                if (N, K) == (256, 1024) and mr <= 3 and fmt != "block_fp8":
                    assert c.kernel == q.KERNEL_STREAM_LDS, (fmt, mr, K, c)
    # (K, N) = (2048, 4096) has no grouped entries either
    assert q.select_grouped_config("fp8", 2, 4096, 2048).kernel == q.KERNEL_GEMV


def test_noalloc_validation_and_workspace_limit():
    lib = q.lib()
    # the scratch-array entry point validates like qlin_scaled_mm, before any HIP call
    args = lambda sc, dt, M, N, K, A=A16, sA=S4, B=B16, sB=S4, Y=Y16: [
        sc, dt, M, N, K, A, K, sA, B, K, sB, Y, N, None]
    assert lib.qlin_scaled_mm_noalloc(*args(5, q.E4M3, 16, 256, 1024)) == ST["arg"]
    assert lib.qlin_scaled_mm_noalloc(*args(q.BLOCK128, q.INT8, 16, 256, 1024)) == ST["arg"]
    assert lib.qlin_scaled_mm_noalloc(*args(q.TOKEN_CHANNEL, q.INT8, 16, 256, 1000)) == ST["shape"]
    assert lib.qlin_scaled_mm_noalloc(*args(q.TOKEN_CHANNEL, q.INT8, 16, 256, 1024, A=None)) == ST["null"]
    assert lib.qlin_scaled_mm_noalloc(*args(q.BLOCK128, q.E4M3, 16, 200, 1024)) == ST["shape"]
    assert lib.qlin_scaled_mm_noalloc(*args(q.TOKEN_CHANNEL, q.E4M3, 0, 256, 1024)) == ST["ok"]
    # a config whose split partials exceed the 32 MiB array: rejected, nothing launched
    fmt, M, N, K = oversize_shape()
    sc, dt = q.FORMATS[fmt]
    assert lib.qlin_scaled_mm_noalloc(*args(sc, dt, M, N, K)) == ST["ws"]


OVERSIZE = [("block_fp8", 2048, 5120, 25600), ("block_fp8", 512, 4096, 12288),
            ("fp8", 1024, 4096, 12288), ("int8", 2048, 5120, 25600), ("fp8", 2048, 5120, 25600)]


def oversize_shape():
    """A shape whose selected config needs more than the 32 MiB scratch array."""
    for fmt, M, N, K in OVERSIZE:
        if q.workspace_size(fmt, M, N, K) > 32 << 20:
            return fmt, M, N, K
    raise AssertionError("no candidate shape needs more than 32 MiB of split-K workspace")


def test_grouped_table_entries(tmp_path):
    # A `grouped` line configures grouped calls only, keyed by the bound on
    # rows per expert (smallest tuned bound >= max_rows, else the largest).
    N, K = 1536, 2048
    path = tmp_path / "t.cfg"
    path.write_text(
        "grouped fp8 1536 2048 4 2 1 8 16 512 1 4 4 1 1\n"
        "grouped fp8 1536 2048 64 1 1 64 128 128 1 4 4 1 1\n"
        "fp8 1536 2048 4 0 1 16 16 512 1 4 2 1 1\n")
    try:
        q.load_config_table(str(path))
        c = q.select_grouped_config("fp8", 3, N, K)
        assert (c.kernel, c.tile_m, c.tile_n) == (q.KERNEL_STREAM_LDS, 8, 16)
        c = q.select_grouped_config("fp8", 5, N, K)
        assert (c.kernel, c.tile_m, c.tile_n) == (q.KERNEL_TILE, 64, 128)
        c = q.select_grouped_config("fp8", 500, N, K)          # past the largest bound
        assert (c.kernel, c.tile_m) == (q.KERNEL_TILE, 64)
        c = q.select_config("fp8", 4, N, K)                    # ordinary calls ignore grouped lines
        assert (c.kernel, c.tile_k) == (q.KERNEL_STREAM, 512)
        # a grouped line with split_k != 1 is malformed: the table is kept
        bad = tmp_path / "bad.cfg"
        bad.write_text("grouped fp8 1536 2048 4 2 1 8 16 512 1 4 4 2 1\n")
        with pytest.raises(q.QlinError):
            q.load_config_table(str(bad))
        assert q.config_table_size() == 3
    finally:
        q.load_config_table(None)


def test_token_stationary_kernel_limits():
    # the persistent token-stationary kernel: its split's token rows must fit
    # 80 KB of LDS, split-K only with the two-pass reduction, never grouped
    tok = [c for c in q.instances_for("int8") if c.kernel == q.KERNEL_STREAM_TOK]
    assert tok and all(c.variant == q.SWAP_AB and c.tile_n == 16 * c.waves_k for c in tok)
    c = [x for x in tok if x.tile_m == 32][0]
    assert q.check_config("int8", 32, 4096, 2560, c) == 0
    assert q.check_config("int8", 32, 4096, 2816, c) != 0
    assert q.check_config("int8", 32, 4096, 5120, c.replace(split_k=2, reduce=q.REDUCE_TWO_PASS)) == 0
    assert q.check_config("int8", 32, 4096, 5120, c.replace(split_k=2, reduce=q.REDUCE_LAST_ARRIVER)) != 0
    assert not [x for x in q.instances_for("block_fp8") if x.kernel == q.KERNEL_STREAM_TOK]
