"""Benchmark of the quantized linear GEMM on one MI355X.

A step is one pass of the hot path over a whole workload: one scaled_mm /
block_scaled_mm call per (format, M, N, K) point, each on the weight matrix
already resident in HBM.  The default workload is the largest decode
configuration: FP8_Dynamic, W8A8_INT8 and Block_FP8 on the 32B-class decoder
linears (K, N) in {(5120,10240), (8192,5120), (5120,51200), (25600,5120)} at
every decode token count M in {1,2,4,8,16,24,32}: 84 GEMMs.  The same line
also reports the W8A8_INT8 1.7B-class decode workload (28 GEMMs) and the
M >= 512 points (TFLOP/s).

Cold caches: every call of a step reads its own copy of the weights, and the
copies rotate over enough steps that about 1 GiB of distinct weights passes
through between two reads of the same copy (a step of the default workload
alone reads 10 GB of weights); the 256 MB Infinity Cache and the L2s cannot
serve them.  The per-point timings
rotate over ~1 GiB of copies of the point's own weights likewise.  A step is captured once into a HIP graph per
rotation set and replayed (graph replay is also how the pages benchmark and
deploy their kernels), so the time is GPU time, not Python launch overhead.

Metric: effective TB/s = algorithmic bytes / time, with algorithmic bytes
M*K + N*K + 2*M*N + scale bytes per GEMM (each operand moved once).

Prints ONE JSON line.  --gpus N with N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_PEAK_TOPS = 5000.0         # MI355X dense fp8 / int8, published (TFLOP/s, TOP/s)

WORKLOAD_TEXT = {
    "int8_1p7b_decode": "W8A8_INT8 scaled_mm, 1.7B-class decoder linears (K,N) in "
                        "{(2048,4096),(2048,2048),(2048,12288),(6144,2048)} x M in {1,2,4,8,16,24,32}",
    "fp8_8b": "FP8_Dynamic scaled_mm, 8B-class linears (K,N) in {(4096,6144),(4096,4096),"
              "(4096,24576),(12288,4096)} x M in {1,2,4,8,16,24,32,128,512}",
    "block_fp8_8b": "Block_FP8 block_scaled_mm, 8B-class linears x M in {1,2,4,8,16,24,32,512}",
    "all_32b": "FP8_Dynamic, W8A8_INT8 and Block_FP8 on 32B-class linears (K,N) in "
               "{(5120,10240),(8192,5120),(5120,51200),(25600,5120)} x M in {1,2,4,8,16,24,32,2048}",
    "all_32b_decode": "FP8_Dynamic, W8A8_INT8 and Block_FP8 on 32B-class linears (K,N) in "
                      "{(5120,10240),(8192,5120),(5120,51200),(25600,5120)} x M in {1,2,4,8,16,24,32}",
    "fp8_small": "FP8_Dynamic scaled_mm, M=16 N=512 K=1024",
    "prefill": "the M >= 512 points: FP8_Dynamic and Block_FP8 8B-class at M=512, all three "
               "formats on the 32B-class linears at M=2048",
}


def alg_bytes(fmt: str, M: int, N: int, K: int) -> int:
    if fmt == "block_fp8":
        scales = 4 * M * (K // 128) + 4 * (N // 128) * (K // 128)
    else:
        scales = 4 * M + 4 * N
    return M * K + N * K + 2 * M * N + scales


def alg_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Workload:
    """Device-resident inputs of every point, with rotating weight copies."""

    def __init__(self, name: str, copies_target_bytes: int = 1 << 30):
        import torch

        import synth
        import int8_gemm_linear_amd as q
        from synth import make_case, make_case_seed0

        self.name = name
        self.points = synth.workload(name)
        dev = torch.device("cuda:0")
        self.dev = dev
        self.q = q
        per_step_b = sum(N * K for (_, _, N, K) in self.points)
        self.sets = max(2, -(-copies_target_bytes // per_step_b))
        self.items = []
        weights = {}
        for (fmt, M, N, K) in self.points:
            case = make_case_seed0(fmt, M, N, K) if (fmt, M, N, K) == ("fp8", 16, 512, 1024) \
                else make_case(fmt, M, N, K)
            dt = torch.int8 if fmt == "int8" else torch.float8_e4m3fn
            a = torch.from_numpy(np.ascontiguousarray(case.A)).to(dev).view(dt)
            sa = torch.from_numpy(np.ascontiguousarray(case.sA)).to(dev)
            key = (fmt, N, K)
            if key not in weights:
                weights[key] = (torch.from_numpy(np.ascontiguousarray(case.B)).to(dev).view(dt),
                                torch.from_numpy(np.ascontiguousarray(case.sB)).to(dev))
            b0, sb = weights[key]
            copies = [b0] + [b0.clone() for _ in range(self.sets - 1)]
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            cfg = q.select_config(fmt, M, N, K)
            self.items.append(dict(fmt=fmt, M=M, N=N, K=K, case=case, a=a, sa=sa, b=copies, sb=sb,
                                   y=y, cfg=cfg, bytes=alg_bytes(fmt, M, N, K),
                                   flops=alg_flops(M, N, K)))
        self.bytes_per_step = sum(it["bytes"] for it in self.items)
        self.flops_per_step = sum(it["flops"] for it in self.items)
        self.weight_bytes = sum(it["N"] * it["K"] * self.sets for it in self.items)

    def call(self, it, s):
        self.call_b(it, it["b"][s])

    def call_b(self, it, b):
        q = self.q
        if it["fmt"] == "block_fp8":
            q.block_scaled_mm(it["a"], it["sa"], b, it["sb"], out=it["y"], config=it["cfg"])
        else:
            q.scaled_mm(it["a"], it["sa"], b, it["sb"], out=it["y"], config=it["cfg"])

    def point_us(self, it, reps: int, cold_bytes: int = 1 << 30, max_copies: int = 256) -> float:
        """Mean launch time of one point: a graph of at least `reps` launches,
        each on the next of enough weight copies (the point's own plus
        temporary clones) that ~`cold_bytes` of distinct weights pass between
        two reads of one copy, so neither the Infinity Cache nor the L2s
        serve the weights; after one untimed replay, three replays each
        timed with events on the launch stream, the median taken (one
        replay's window can catch the GPU in another state)."""
        import torch
        n = int(min(max_copies, max(len(it["b"]), -(-cold_bytes // (it["N"] * it["K"])))))
        bs = list(it["b"]) + [it["b"][0].clone() for _ in range(n - len(it["b"]))]
        launches = max(reps, n)
        g = capture(lambda: [self.call_b(it, bs[r % n]) for r in range(launches)])
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / launches)
        del g, bs
        return float(np.median(ts))

    def step(self, s):
        for it in self.items:
            self.call(it, s)


def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def run_gpu(wl: Workload, steps: int, warmup: int, reps: int, points: bool = True):
    import torch

    for i in range(max(1, warmup)):
        wl.step(i % wl.sets)
    torch.cuda.synchronize()
    graphs = [capture(lambda s=s: wl.step(s)) for s in range(wl.sets)]
    for i in range(max(1, warmup)):
        graphs[i % wl.sets].replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        graphs[i % wl.sets].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)

    # ---- per-kernel durations, each point on its own with cold weights
    per = [wl.point_us(it, reps) for it in wl.items] if points else []
    torch.cuda.empty_cache()
    return ms, per


def cpu_baseline(wl: Workload, threads: int, budget_s: float):
    """The oracle on the workload's points: whole points, in order, in repeated
    passes until the time budget is spent.  Also returns the oracle outputs of
    the first pass for a parity check of the GPU outputs."""
    import oracle
    from tests import parity as par

    done_bytes = 0
    done_flops = 0
    n_calls = 0
    first = []
    t0 = time.perf_counter()
    while True:
        for it in wl.items:
            case = it["case"]
            ref = oracle.scaled_mm(par.FMT_CODE[case.fmt], case.A, case.sA, case.B, case.sB,
                                   block=case.block, nthreads=threads)
            done_bytes += it["bytes"]
            done_flops += it["flops"]
            n_calls += 1
            if len(first) < len(wl.items):
                first.append((it, ref))
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    secs = time.perf_counter() - t0
    return done_bytes, done_flops, secs, n_calls, first


def prefill_points(reps: int = 4):
    """Per-point GEMM time of the MFMA-bound (M >= 512) points, each with
    cold weights (Workload.point_us: at least `reps` launches rotating over
    ~1 GiB of weight copies, at most 64 of them)."""
    import torch
    wl = Workload("prefill", copies_target_bytes=0)
    for it in wl.items:                # eager calls size the split-K workspace before capture
        wl.call(it, 0)
    torch.cuda.synchronize()
    out = []
    for it in wl.items:
        us = wl.point_us(it, reps, max_copies=64)
        torch.cuda.empty_cache()
        tf = it["flops"] / us / 1e6
        c = it["cfg"]
        out.append({"fmt": it["fmt"], "M": it["M"], "N": it["N"], "K": it["K"], "us": round(us, 2),
                    "tflops": round(tf, 1), "frac": round(tf / MFMA_PEAK_TOPS, 4),
                    "cfg": f"k{c.kernel} v{c.variant} {c.tile_m}x{c.tile_n}x{c.tile_k} "
                           f"w{c.waves_n}x{c.waves_k} s{c.stages} split{c.split_k}"})
    del wl
    torch.cuda.empty_cache()
    tfs = np.array([p["tflops"] for p in out])
    geo = float(np.exp(np.log(tfs).mean()))
    return {"unit": "TFLOP/s", "peak": MFMA_PEAK_TOPS, "geomean_tflops": round(geo, 1),
            "geomean_frac": round(geo / MFMA_PEAK_TOPS, 4), "min_frac": round(float(tfs.min()) / MFMA_PEAK_TOPS, 4),
            "max_frac": round(float(tfs.max()) / MFMA_PEAK_TOPS, 4), "points": out}


# Activation producers upstream of the GEMM (quantizers and fused norm /
# activation + quantizer), at the decode (M = 32) and prefill (M = 2048)
# sizes of the 8B- and 32B-class models, plus SiLU-and-mul at the decode
# size of the 1.7B-class model (intermediate 6144): (op, M, K).  Algorithmic
# bytes: every input and output moved once (bf16 2 B, codes 1 B, fp32 scales).
PRODUCER_POINTS = [
    ("quant_per_token", 32, 4096), ("quant_per_token", 2048, 5120),
    ("quant_per_group128", 2048, 5120),
    ("rms_norm_dynamic_per_token_quant", 32, 4096), ("rms_norm_dynamic_per_token_quant", 2048, 5120),
    ("rms_norm_per_block_quant", 2048, 5120),
    ("silu_and_mul_dynamic_per_token_quant", 32, 6144),
    ("silu_and_mul_dynamic_per_token_quant", 32, 12288),
    ("silu_and_mul_dynamic_per_token_quant", 2048, 25600),
    ("silu_and_mul_per_block_quant", 2048, 25600),
]


def producer_bytes(op: str, M: int, K: int) -> int:
    group = "group" in op or "block" in op
    scales = 4 * M * (K // 128) if group else 4 * M
    if op.startswith("rms_norm"):
        return 2 * M * K * 3 + 2 * K + M * K + scales     # x, residual in/out, weight, codes
    if op.startswith("silu"):
        return 4 * M * K + M * K + scales                 # gate | up, codes
    return 2 * M * K + M * K + scales


def producer_points(reps: int = 8, target_bytes: int = 1 << 30):
    """Per-call time of the producers: a graph of `reps` launches per point,
    rotating over enough input copies that ~1 GiB passes between two reads
    of the same copy (cold caches), timed with events on the launch stream."""
    import torch
    import int8_gemm_linear_amd as q
    import synth
    dev = torch.device("cuda:0")
    out = []
    for op, M, K in PRODUCER_POINTS:
        cols = 2 * K if op.startswith("silu") else K
        x0 = torch.from_numpy(synth.activations(M, cols, (51, 2, M, cols), outliers=True,
                                                outlier_key=(51, 3, cols))).to(dev).to(torch.bfloat16)
        nb = producer_bytes(op, M, K)
        copies = max(2, min(64, -(-target_bytes // nb)))
        xs = [x0] + [x0.clone() for _ in range(copies - 1)]
        rs = [x.clone() for x in xs] if op.startswith("rms_norm") else None
        w = torch.from_numpy(synth.norm_weight(K, (51, 4, K))).to(dev).to(torch.bfloat16)
        codes = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
        sc = torch.empty((M, K // 128) if ("group" in op or "block" in op) else (M,),
                         dtype=torch.float32, device=dev)

        def call(i, op=op, xs=xs, rs=rs, w=w, codes=codes, sc=sc):
            x = xs[i % len(xs)]
            if op == "quant_per_token":
                q.quant_per_token(x, out=codes, scale=sc)
            elif op == "quant_per_group128":
                q.quant_per_group128(x, out=codes, scale=sc)
            elif op == "rms_norm_dynamic_per_token_quant":
                q.rms_norm_dynamic_per_token_quant(x, w, 1e-6, residual=rs[i % len(rs)], out=codes,
                                                   scale=sc)
            elif op == "rms_norm_per_block_quant":
                q.rms_norm_per_block_quant(x, w, 1e-6, residual=rs[i % len(rs)], out=codes, scale=sc)
            elif op == "silu_and_mul_dynamic_per_token_quant":
                q.silu_and_mul_dynamic_per_token_quant(x, out=codes, scale=sc)
            else:
                q.silu_and_mul_per_block_quant(x, out=codes, scale=sc)

        n = max(reps, copies)
        call(0)
        torch.cuda.synchronize()
        g = capture(lambda: [call(i) for i in range(n)])
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / n
        del g, xs, rs
        gbs = nb / us / 1e3
        out.append({"op": op, "M": M, "K": K, "us": round(us, 2), "alg_bytes": nb,
                    "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)})
    torch.cuda.empty_cache()
    return {"unit": "GB/s", "peak": HBM_PEAK_GBS, "timing": "HIP-graph replay, rotating input "
            "copies (~1 GiB between reuses), hipEvents", "points": out}


MOE_BATCHES = [1, 32, 512]


def moe_points(reps: int = 8, target_bytes: int = 1 << 30):
    """One grouped launch per MoE layer call (device offset table), timed
    from a graph over rotating weight copies; beside it the same work as one
    scaled_mm launch per active expert (captured likewise) for comparison.
    Algorithmic bytes: each active expert's weights and scales once, its
    token rows and outputs once."""
    import torch
    import int8_gemm_linear_amd as q
    import synth
    dev = torch.device("cuda:0")
    out = []
    for name, K, N in synth.MOE_LAYERS:
        E = synth.MOE_EXPERTS
        w = torch.from_numpy(np.ascontiguousarray(
            synth.rng(81, K, N).integers(0, 0x7E, (E, N, K), dtype=np.uint8) |
            (synth.rng(82, K, N).integers(0, 2, (E, N, K), dtype=np.uint8) << 7))).to(dev)
        w = w.view(torch.float8_e4m3fn)
        sb = torch.full((E, N), 1e-3, dtype=torch.float32, device=dev)
        copies = max(2, -(-target_bytes // (E * N * K)))
        ws = [w] + [w.clone() for _ in range(copies - 1)]
        for B in MOE_BATCHES:
            counts = synth.moe_counts(B, K)
            rows = int(counts.sum())
            off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
            a = torch.from_numpy(synth.rng(84, B, K).integers(0, 0x7E, (rows, K), dtype=np.uint8)).to(dev)
            a = a.view(torch.float8_e4m3fn)
            sa = torch.full((rows,), 1e-2, dtype=torch.float32, device=dev)
            y = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
            max_rows = int(counts.max())
            n = max(reps, copies)

            def grouped(i):
                q.grouped_scaled_mm(a, sa, ws[i % copies], sb, off, max_rows, out=y)

            act = [e for e in range(E) if counts[e] > 0]
            starts = np.concatenate([[0], np.cumsum(counts)])

            def loop(i):
                wi = ws[i % copies]
                for e in act:
                    lo, hi = int(starts[e]), int(starts[e + 1])
                    q.scaled_mm(a[lo:hi], sa[lo:hi], wi[e], sb[e], out=y[lo:hi])

            def timed(fn, calls):
                fn(0)
                torch.cuda.synchronize()
                gr = capture(lambda: [fn(i) for i in range(calls)])
                gr.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                gr.replay()
                e1.record()
                torch.cuda.synchronize()
                del gr
                return e0.elapsed_time(e1) * 1e3 / calls

            us = timed(grouped, n)
            loop_us = timed(loop, min(n, 4))
            nb = len(act) * (N * K + 4 * N) + rows * (K + 2 * N + 4)
            cfg = q.select_grouped_config("fp8", max_rows, N, K)
            out.append({"layer": name, "K": K, "N": N, "batch": B, "experts_active": len(act),
                        "rows": rows, "max_rows": max_rows, "us": round(us, 2), "alg_bytes": nb,
                        "tbs": round(nb / us / 1e6, 3), "frac": round(nb / us / 1e6 / 8.0, 4),
                        "tflops": round(2.0 * rows * N * K / us / 1e6, 1),
                        "per_expert_launches_us": round(loop_us, 2),
                        "cfg": f"k{cfg.kernel} v{cfg.variant} {cfg.tile_m}x{cfg.tile_n}x{cfg.tile_k} "
                               f"w{cfg.waves_n}x{cfg.waves_k} s{cfg.stages} split1"})
        del ws, w
        torch.cuda.empty_cache()
    return {"unit": "TB/s", "peak_tbs": 8.0, "model": "128 experts, top-8, hidden 2048, expert width 768",
            "timing": "HIP-graph replay, rotating weight copies (>= 1 GiB), hipEvents", "points": out}


def cpu_model() -> str:
    """The host CPU's model name, with its family / model / stepping numbers
    (some hosts report only a generic name)."""
    name, ids = "unknown", {}
    try:
        for ln in open("/proc/cpuinfo"):
            key, _, val = ln.partition(":")
            key = key.strip()
            if key == "model name" and name == "unknown":
                name = val.strip()
            elif key in ("cpu family", "model", "stepping") and key not in ids:
                ids[key] = val.strip()
            elif not ln.strip() and name != "unknown":
                break
    except OSError:
        pass
    if ids:
        name += " (family %s, model %s, stepping %s)" % (
            ids.get("cpu family", "?"), ids.get("model", "?"), ids.get("stepping", "?"))
    return name


def dispatch_cost():
    """Host-side dispatch cost of the C ABI (int8_gemm_linear_amd/qlin_dispatch_bench,
    built with the library): one JSON object, or None when it is not built."""
    import subprocess
    exe = os.path.join(ROOT, "int8_gemm_linear_amd", "qlin_dispatch_bench")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        log("dispatch bench failed:", r.stderr[-300:])
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def load_traffic(workload: str, table: str | None):
    """HBM bytes per GEMM call from the committed counter record of this
    workload, or None when the kernels or the table changed since."""
    from int8_gemm_linear_amd import profsum
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None, "no counter record"
    with open(path) as f:
        rec = json.load(f)
    if rec.get("fingerprint") != profsum.fingerprint(table):
        return None, "kernels or table changed since the counters were taken"
    return rec["traffic_bytes_per_call"], os.path.relpath(path, ROOT)


def oracle_threads() -> tuple[int, dict]:
    """Threads for the oracle timing: every host CPU this process may run on,
    capped by OMP_NUM_THREADS when set (the host's CPU share per GPU)."""
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = nproc
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = avail
    if cap and cap.isdigit() and int(cap) > 0:
        threads = min(threads, int(cap))
    return max(1, threads), {"nproc": nproc, "affinity_cpus": avail, "omp_num_threads": cap}


def step_timing(wl: "Workload", steps: int, warmup: int, reps: int, points: bool):
    """Time `steps` steps of a workload; returns a dict of the step-level figures
    plus the per-point launch times (empty without points)."""
    ms, per_us = run_gpu(wl, steps, warmup, reps, points=points)
    ms_step = ms / steps
    n_launch = len(wl.items)
    launch_bytes = wl.bytes_per_step / n_launch
    launch_us = ms_step * 1e3 / n_launch
    return {"ms_step": ms_step, "value_tbs": wl.bytes_per_step / (ms_step * 1e-3) / 1e12,
            "launch_bytes": launch_bytes, "launch_us": launch_us,
            "achieved_gbs": launch_bytes / (launch_us * 1e-6) / 1e9,
            "flops_tops": wl.flops_per_step / (ms_step * 1e-3) / 1e12}, per_us


def per_format(wl: "Workload", per_us) -> dict:
    """TB/s and fraction of 8 TB/s per format, from the per-point times."""
    out = {}
    for fmt in ("fp8", "int8", "block_fp8"):
        pts = [(it, us) for it, us in zip(wl.items, per_us) if it["fmt"] == fmt]
        if not pts:
            continue
        b = sum(it["bytes"] for it, _ in pts)
        t = sum(us for _, us in pts)
        tbs = b / t / 1e6
        geo = float(np.exp(np.mean([np.log(it["bytes"] / us / 1e6) for it, us in pts])))
        out[fmt] = {"points": len(pts), "tbs": round(tbs, 4), "frac": round(tbs / 8.0, 4),
                    "geomean_tbs": round(geo, 4), "sum_us": round(t, 2)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all_32b_decode", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--reps", type=int, default=24, help="launches per point in the kernel-timing graphs")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one 256 MiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--table", default=None, help="config table file to load before running")
    ap.add_argument("--per-point", action="store_true", help="print per-point timings to stderr")
    ap.add_argument("--no-points", action="store_true",
                    help="skip the per-point timings (counter runs: every point then "
                         "launches equally often, as in a step)")
    ap.add_argument("--no-dispatch", action="store_true", help="skip the host dispatch-cost run")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M >= 512 per-point timings")
    ap.add_argument("--no-moe", action="store_true", help="skip the grouped (MoE) GEMM timings")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the activation-producer timings (quantizers, fused norm / SiLU)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the W8A8_INT8 1.7B-class decode workload reported beside the headline")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note, not a code path)"}))
        sys.exit(2)

    import torch
    import int8_gemm_linear_amd as q

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    q.lib()
    if args.table:
        q.load_config_table(args.table)
    wl = Workload(args.workload)
    log(f"workload {args.workload}: {len(wl.items)} GEMMs/step, {wl.bytes_per_step / 1e6:.1f} MB "
        f"algorithmic/step, {wl.sets} weight copies ({wl.weight_bytes / 2**30:.2f} GiB)")
    head, per_us = step_timing(wl, args.steps, args.warmup, args.reps, points=not args.no_points)
    log(f"step {head['ms_step'] * 1e3:.1f} us, {head['value_tbs']:.3f} TB/s")
    kern_us = sum(per_us)
    traffic, traffic_src = load_traffic(args.workload, args.table)
    if args.per_point:
        for it, us in zip(wl.items, per_us):
            c = it["cfg"]
            log(f"  {it['fmt']:9s} M={it['M']:5d} N={it['N']:6d} K={it['K']:6d}  {us:8.2f} us  "
                f"{it['bytes'] / us / 1e6:7.3f} TB/s  {it['flops'] / us / 1e6:8.1f} TFLOP/s  "
                f"k={c.kernel} v={c.variant} t={c.tile_m}x{c.tile_n}x{c.tile_k} "
                f"w={c.waves_n}x{c.waves_k} st={c.stages} s={c.split_k} r={c.reduce}")

    if args.copy_calib:
        # a plain elementwise copy of known size: reads 256 MiB, writes 256 MiB
        src = torch.zeros(64 << 20, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    parity_ok = None
    if not args.no_cpu:
        from tests import parity as par
        threads, host = oracle_threads()
        done_bytes, done_flops, secs, n_calls, first = cpu_baseline(wl, threads, args.cpu_budget)
        # the GPU outputs of the last replayed step vs the oracle
        parity_ok = True
        for it, ref in first:
            try:
                par.check_y(it["fmt"], par.y_bits(it["y"]), ref.y, ref.ydbl, ref.bound)
            except AssertionError as e:
                parity_ok = False
                log("PARITY FAIL", it["fmt"], it["M"], it["N"], it["K"], str(e)[:200])
        b1, _, s1, n1, _ = cpu_baseline(wl, 1, args.cpu_budget / 3)
        cpu = {"value": done_bytes / secs / 1e12, "unit": "TB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{n_calls} GEMM calls ({n_calls / len(wl.items):.2f} passes over the "
                         f"{len(wl.items)} GEMMs of the workload, in order, whole GEMMs), {secs:.1f} s "
                         f"on {threads} threads (plain C, double/int64 accumulate)",
               "single_thread_value": b1 / s1 / 1e12,
               "single_thread_sample": f"{n1} GEMM calls, {s1:.1f} s on 1 thread",
               "gflops": round(done_flops / secs / 1e9, 2),
               "host_cpu": cpu_model(), **host,
               "parity_checked_gemms": len(first)}
    points_fmt = per_format(wl, per_us) if per_us else None
    wl_items = len(wl.items)
    wl_bytes = wl.bytes_per_step
    del wl
    torch.cuda.empty_cache()

    extra = None
    if not args.no_extra and args.workload != "int8_1p7b_decode":
        w2 = Workload("int8_1p7b_decode")
        e, per2 = step_timing(w2, args.steps, args.warmup, args.reps, points=not args.no_points)
        extra = {"workload": WORKLOAD_TEXT["int8_1p7b_decode"], "gemms_per_step": len(w2.items),
                 "value": round(e["value_tbs"], 4), "unit": "TB/s", "ms_per_step": round(e["ms_step"], 5),
                 "launch_avg_us": round(e["launch_us"], 3),
                 "frac": round(e["achieved_gbs"] / HBM_PEAK_GBS, 4),
                 "isolated_launch_avg_us": round(sum(per2) / len(per2), 3) if per2 else None}
        del w2
        torch.cuda.empty_cache()

    dispatch = None if args.no_dispatch else dispatch_cost()
    prefill = None
    if not args.no_prefill and args.workload != "prefill":
        prefill = prefill_points()

    producers = None
    if not args.no_producers and args.workload != "prefill":
        producers = producer_points()
    moe = None
    if not args.no_moe and args.workload != "prefill":
        moe = moe_points()

    fmts = {it[0] for it in synth_points(args.workload)}
    out = {
        "metric": "effective TB/s (M<=32) and TFLOPS (M>=512) for FP8/INT8 scaled GEMM, 1 GPU",
        "value": round(head["value_tbs"], 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if fmts == {"int8"} else "e4m3/int8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "gemms_per_step": wl_items,
                   "alg_bytes_per_step": wl_bytes, "tflops": round(head["flops_tops"], 2),
                   "timing": "HIP-graph replay of whole steps, hipEvents, cold weights"},
        "roofline": {"bound": "hbm", "achieved": round(head["achieved_gbs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "the GEMM launch (kernel instance per shape from the tuned table); "
                               "algorithmic bytes per launch = mean over the step's GEMMs",
                     "alg_bytes_per_launch": round(head["launch_bytes"], 1),
                     "launch_avg_us": round(head["launch_us"], 3),
                     "isolated_launch_avg_us": round(kern_us / len(per_us), 3) if per_us else None,
                     "traffic_src": traffic_src},
        "per_format": points_fmt,
        "cpu_baseline": cpu,
        "int8_1p7b_decode": extra,
        "dispatch": dispatch,
        "prefill_mfma": prefill,
        "producers": producers,
        "moe_grouped": moe,
        "parity_vs_oracle": parity_ok,
    }
    print(json.dumps(out), flush=True)


def synth_points(name: str):
    import synth
    return synth.workload(name)


if __name__ == "__main__":
    main()
