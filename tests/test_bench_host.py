"""Host-side checks of the benchmark (CPU only): the workload it times, the
algorithmic byte and flop counts its metrics divide by, the one-GPU guard
and the counter-record fingerprint rule.  Nothing here touches a GPU."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_default_workload_is_the_28_decode_gemms():
    # W8A8_INT8 on the 1.7B-class linears (K, N) x the decode token grid
    pts = synth.workload("int8_1p7b_decode")
    assert len(pts) == 28
    assert {p[0] for p in pts} == {"int8"}
    assert {(K, N) for (_, _, N, K) in pts} == {(2048, 4096), (2048, 2048), (2048, 12288),
                                                 (6144, 2048)}
    assert sorted({M for (_, M, _, _) in pts}) == [1, 2, 4, 8, 16, 24, 32]


def test_prefill_workload_is_every_point_with_512_or_more_tokens():
    pts = synth.workload("prefill")
    assert pts and all(M >= 512 for (_, M, _, _) in pts)
    every = [p for w in ("fp8_8b", "block_fp8_8b", "all_32b") for p in synth.workload(w)]
    assert sorted(pts) == sorted(p for p in every if p[1] >= 512)


def test_algorithmic_bytes_count_every_operand_once():
    # token/channel: A (M*K) + B (N*K) + bf16 Y (2*M*N) + fp32 scales 4*(M+N)
    assert bench.alg_bytes("int8", 1, 2048, 2048) == 2048 + 2048 * 2048 + 2 * 2048 + 4 * (1 + 2048)
    assert bench.alg_bytes("fp8", 32, 4096, 2048) == 32 * 2048 + 4096 * 2048 + 2 * 32 * 4096 + 4 * (32 + 4096)
    # block: one fp32 scale per 1x128 activation group and per 128x128 weight block
    M, N, K = 16, 512, 1024
    assert bench.alg_bytes("block_fp8", M, N, K) == (M * K + N * K + 2 * M * N
                                                     + 4 * M * (K // 128) + 4 * (N // 128) * (K // 128))
    assert bench.alg_flops(2048, 51200, 5120) == 2 * 2048 * 51200 * 5120


def test_step_bytes_of_the_default_workload():
    # 357,528,944 algorithmic bytes per step: the figure the headline TB/s divides by
    total = sum(bench.alg_bytes(f, M, N, K) for (f, M, N, K) in synth.workload("int8_1p7b_decode"))
    assert total == 357528944


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_record_is_dropped_when_the_kernels_change(tmp_path):
    # the committed counter record is used only while its fingerprint (kernel
    # sources + config table) matches the tree; another table changes it
    from int8_gemm_linear_amd import profsum
    rec = os.path.join(ROOT, "profiles", "int8_1p7b_decode_traffic.json")
    assert os.path.exists(rec)
    other = tmp_path / "table.cfg"
    other.write_text("# empty table\n")
    assert profsum.fingerprint(str(other)) != profsum.fingerprint(None)
    traffic, why = bench.load_traffic("int8_1p7b_decode", str(other))
    assert traffic is None and "changed" in why


def test_producer_bytes_count_every_operand_once():
    # per value: bf16 input 2 B, code 1 B; SiLU-and-mul reads gate and up
    # (4 B); the RMS norm also reads and writes the residual (2 + 2 B) and
    # reads the bf16 weight once; fp32 scales per row or per 1x128 group
    M, K = 32, 4096
    row_scales, group_scales = 4 * M, 4 * M * (K // 128)
    assert bench.producer_bytes("quant_per_token", M, K) == 3 * M * K + row_scales
    assert bench.producer_bytes("quant_per_group128", M, K) == 3 * M * K + group_scales
    assert bench.producer_bytes("rms_norm_dynamic_per_token_quant", M, K) == (
        7 * M * K + 2 * K + row_scales)
    assert bench.producer_bytes("rms_norm_per_block_quant", M, K) == 7 * M * K + 2 * K + group_scales
    assert bench.producer_bytes("silu_and_mul_dynamic_per_token_quant", M, K) == 5 * M * K + row_scales
    assert bench.producer_bytes("silu_and_mul_per_block_quant", M, K) == 5 * M * K + group_scales
    # every producer the bench line times is one of these
    assert {op for (op, _, _) in bench.PRODUCER_POINTS} == {
        "quant_per_token", "quant_per_group128", "rms_norm_dynamic_per_token_quant",
        "rms_norm_per_block_quant", "silu_and_mul_dynamic_per_token_quant",
        "silu_and_mul_per_block_quant"}
