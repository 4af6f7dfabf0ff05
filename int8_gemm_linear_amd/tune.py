"""Offline per-shape tuning sweep on the MI355X.

The pages replace hand-written dispatch rules (for instance "use Swap-AB
below 32 tokens") by a per-shape ahead-of-time search over the algorithm
variant and the low-level launch configuration ("Building a High-Performance
and Portable vLLM Linear Backend with Helion", section "Kernel
Implementation"; the techfeed.io summary gives the tunable domains, split_k a
power of two in [1, 256] and swap_ab a boolean).  Our search space is small
enough to sweep exhaustively: every built kernel instance x variant x split_k
x reduction mode that is valid for the shape.

Each candidate is timed as the pages time theirs, under graph replay: a HIP
graph of R launches, each on a different copy of the weights (together
larger than the 256 MB Infinity Cache, so weights come from HBM), replayed a
few times; the per-launch time is the median replay time / R.  A candidate
whose output differs from the reference candidate's is discarded (INT8: bit
for bit; FP8: a normwise difference above 1e-2, or an element further than
2^-5 of the output's largest magnitude).

    python -m int8_gemm_linear_amd.tune --workload int8_1p7b_decode \
        --jsonl tune.jsonl --table int8_gemm_linear_amd/configs/qlin_mi355x.cfg

Results are appended to the JSONL log and a restart skips finished
(point, candidate) pairs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import int8_gemm_linear_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COLD_BYTES = 512 << 20


def candidates(fmt: str, M: int, N: int, K: int, max_split: int = 256, kernels=None,
               max_token_tiles: int = 4):
    """Every valid (instance, split_k, reduce) for the point; `kernels`
    restricts the kernel families, `max_token_tiles` the token tiles of the
    stream kernels (ceil(M / tile_m))."""
    out = []
    KS = -(-K // 128)
    for base in q.instances_for(fmt):
        if kernels is not None and base.kernel not in kernels:
            continue
        lds_ring = base.kernel in (q.KERNEL_STREAM_LDS, q.KERNEL_STREAM_TOK)
        if (base.kernel == q.KERNEL_STREAM or lds_ring) and -(-M // base.tile_m) > max_token_tiles:
            continue                      # the stream kernels are for small token counts
        if lds_ring and base.tile_m > 2 * M and base.tile_m > 4:
            continue                      # a token tile mostly of padding
        if base.kernel == q.KERNEL_TILE and M < 16:
            continue
        if base.kernel == q.KERNEL_GEMV and M > base.tile_m:
            continue                      # one token tile per workgroup column
        split = 1
        while split <= min(max_split, 256):
            kw = base.waves_k if base.kernel == q.KERNEL_STREAM else 1
            if split * kw > KS or (lds_ring and split * 2 > KS):
                break
            reds = (q.REDUCE_LAST_ARRIVER,) if split == 1 else (q.REDUCE_LAST_ARRIVER, q.REDUCE_TWO_PASS)
            for r in reds:
                c = base.replace(split_k=split, reduce=r)
                if q.check_config(fmt, M, N, K, c) == 0:
                    out.append(c)
            split *= 2
    return out


class Point:
    """Device inputs of one (fmt, M, N, K) with enough weight copies to be cold."""

    def __init__(self, fmt, M, N, K, cold_bytes=COLD_BYTES, root=0):
        sys.path.insert(0, ROOT)
        import synth
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        case = synth.make_case(fmt, M, N, K, root=root)
        dt = torch.int8 if fmt == "int8" else torch.float8_e4m3fn
        dev = torch.device("cuda")
        self.a = torch.from_numpy(np.ascontiguousarray(case.A)).to(dev).view(dt)
        self.sa = torch.from_numpy(np.ascontiguousarray(case.sA)).to(dev)
        b = torch.from_numpy(np.ascontiguousarray(case.B)).to(dev).view(dt)
        self.sb = torch.from_numpy(np.ascontiguousarray(case.sB)).to(dev)
        ncopy = int(min(256, max(2, -(-cold_bytes // (N * K)))))
        self.b = [b] + [b.clone() for _ in range(ncopy - 1)]
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = max(q.workspace_size(fmt, M, N, K, c) for c in candidates(fmt, M, N, K)) \
            if M > 0 else 0
        self.ws = torch.zeros(max(ws, 1 << 20), dtype=torch.uint8, device=dev)

    def call(self, cfg, i=0, out=None):
        f = q.block_scaled_mm if self.fmt == "block_fp8" else q.scaled_mm
        return f(self.a, self.sa, self.b[i % len(self.b)], self.sb, out=self.y if out is None else out,
                 config=cfg, workspace=self.ws)

    def time(self, cfg, reps: int | None = None, replays: int = 3) -> float:
        """Median per-launch microseconds over `replays` replays of an R-launch graph."""
        R = reps or len(self.b)
        self.call(cfg)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                self.call(cfg, i)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(replays):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / R)
        del g
        return float(np.median(ts))


class GroupedPoint:
    """Device inputs of one grouped (mixture-of-experts) layer call: E experts'
    weights [E, N, K] (random finite codes, enough copies to be cold), the
    token rows of a batch routed top-k by the seeded uniform routing and
    sorted by expert, and the device offset table."""

    def __init__(self, fmt, N, K, batch, cold_bytes=COLD_BYTES):
        sys.path.insert(0, ROOT)
        import synth
        self.fmt, self.N, self.K, self.batch = fmt, N, K, batch
        E = synth.MOE_EXPERTS
        dev = torch.device("cuda")
        counts = synth.moe_counts(batch, K)
        self.rows = int(counts.sum())
        self.M = int(counts.max())                       # the rows-per-expert bound
        self.off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
        dt = torch.int8 if fmt == "int8" else torch.float8_e4m3fn
        codes = synth.e4m3_codes((E, N, K), (91, K, N))
        if fmt == "int8":
            codes = (codes.view(np.int8) // 2).view(np.uint8)
        b = torch.from_numpy(codes).to(dev).view(dt)
        a = synth.e4m3_codes((self.rows, K), (92, batch, K))
        self.a = torch.from_numpy((a.view(np.int8) // 2).view(np.uint8) if fmt == "int8" else a).to(dev).view(dt)
        if fmt == "block_fp8":
            self.sa = torch.full((self.rows, K // 128), 1e-2, device=dev)
            self.sb = torch.full((E, N // 128, K // 128), 1e-3, device=dev)
        else:
            self.sa = torch.full((self.rows,), 1e-2, device=dev)
            self.sb = torch.full((E, N), 1e-3, device=dev)
        ncopy = int(min(16, max(2, -(-cold_bytes // (E * N * K)))))
        self.b = [b] + [b.clone() for _ in range(ncopy - 1)]
        self.y = torch.empty((self.rows, N), dtype=torch.bfloat16, device=dev)

    def call(self, cfg, i=0, out=None):
        f = q.grouped_block_scaled_mm if self.fmt == "block_fp8" else q.grouped_scaled_mm
        return f(self.a, self.sa, self.b[i % len(self.b)], self.sb, self.off, self.M,
                 out=self.y if out is None else out, config=cfg)

    time = Point.time


def grouped_candidates(fmt, M, N, K):
    """Configs a grouped call can run: split_k = 1 (grid.z is the expert),
    stream-kernel tiles of at most 4 token tiles, no spread placement."""
    return [c for c in candidates(fmt, M, N, K, max_split=1)
            if not (c.kernel == q.KERNEL_STREAM_LDS and c.waves_n == 2)
            and c.kernel != q.KERNEL_STREAM_TOK]


def agree(fmt, y, ref) -> bool:
    """Sanity check of a candidate against the reference candidate (parity
    itself is established by the tests against the oracle).  INT8: bit for
    bit.  FP8: accumulation order differs between candidates, so compare
    normwise and against the output's scale, not elementwise-relative
    (outputs near a cancellation have no meaningful relative error)."""
    if fmt == "int8":
        return torch.equal(y.view(torch.int16), ref.view(torch.int16))
    yf, rf = y.float(), ref.float()
    if not torch.isfinite(yf).all():
        return False
    d = (yf - rf).abs()
    scale = rf.abs().max().item()
    nrm = torch.linalg.vector_norm(rf).item()
    return bool(d.max().item() <= 2.0 ** -5 * scale
                and (torch.linalg.vector_norm(yf - rf).item() <= 1e-2 * nrm or nrm == 0))


def tune_point(fmt, M, N, K, log=None, done=None, max_cands=None, verbose=False, **sel):
    """Times every candidate of the point (`sel`: the filters of candidates());
    the config the library selects now is always among them."""
    pt = Point(fmt, M, N, K)
    cands = candidates(fmt, M, N, K, **sel)
    if max_cands:
        cands = cands[:max_cands]
    cur = q.select_config(fmt, M, N, K)
    if cur not in cands:
        cands = [cur] + cands
    ref = pt.call(q.select_config(fmt, M, N, K), out=torch.empty_like(pt.y)).clone()
    torch.cuda.synchronize()
    results = []
    for c in cands:
        key = json.dumps([fmt, M, N, K, list(c.__dict__.values())])
        if done is not None and key in done:
            results.append((done[key]["us"], c, done[key]["ok"]))
            continue
        y = pt.call(c, out=torch.full_like(pt.y, float("nan")))
        torch.cuda.synchronize()
        ok = agree(fmt, y, ref)
        us = pt.time(c) if ok else float("inf")
        results.append((us, c, ok))
        if log is not None:
            log.write(json.dumps({"key": key, "fmt": fmt, "M": M, "N": N, "K": K,
                                  "cfg": c.__dict__, "us": us, "ok": ok}) + "\n")
            log.flush()
        if verbose:
            print(f"  {us:9.2f} us ok={ok} {c}", flush=True)
    results.sort(key=lambda r: r[0])
    del pt
    torch.cuda.empty_cache()
    return results


def tune_grouped(fmt, N, K, batch, log=None, done=None, verbose=False):
    """Times every grouped candidate of one layer call; returns (results, max_rows)."""
    pt = GroupedPoint(fmt, N, K, batch)
    M = pt.M
    cands = grouped_candidates(fmt, M, N, K)
    cur = q.select_grouped_config(fmt, M, N, K)
    if cur not in cands:
        cands = [cur] + cands
    ref = pt.call(cur, out=torch.empty_like(pt.y)).clone()
    torch.cuda.synchronize()
    results = []
    for c in cands:
        key = json.dumps(["grouped", fmt, batch, N, K, list(c.__dict__.values())])
        if done is not None and key in done:
            results.append((done[key]["us"], c, done[key]["ok"]))
            continue
        y = pt.call(c, out=torch.full_like(pt.y, float("nan")))
        torch.cuda.synchronize()
        ok = agree(fmt, y, ref)
        us = pt.time(c) if ok else float("inf")
        results.append((us, c, ok))
        if log is not None:
            log.write(json.dumps({"key": key, "grouped": True, "fmt": fmt, "batch": batch, "M": M,
                                  "N": N, "K": K, "cfg": c.__dict__, "us": us, "ok": ok}) + "\n")
            log.flush()
        if verbose:
            print(f"  {us:9.2f} us ok={ok} {c}", flush=True)
    results.sort(key=lambda r: r[0])
    del pt
    torch.cuda.empty_cache()
    return results, M


def table_line(fmt, M, N, K, c, grouped=False) -> str:
    return (("grouped " if grouped else "") +
            f"{fmt} {N} {K} {M} {c.kernel} {c.variant} {c.tile_m} {c.tile_n} {c.tile_k} "
            f"{c.waves_n} {c.waves_k} {c.stages} {c.split_k} {c.reduce}")


def alg_bytes(fmt, M, N, K):
    s = 4 * M * (K // 128) + 4 * (N // 128) * (K // 128) if fmt == "block_fp8" else 4 * (M + N)
    return M * K + N * K + 2 * M * N + s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", action="append", default=[])
    ap.add_argument("--point", action="append", default=[], help="fmt,M,N,K")
    ap.add_argument("--jsonl", default=None)
    ap.add_argument("--table", default=None, help="write/merge the best configs into this table")
    ap.add_argument("--max-cands", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--min-m", type=int, default=0)
    ap.add_argument("--max-m", type=int, default=1 << 30)
    ap.add_argument("--kernels", default=None, help="comma list of kernel families to sweep "
                    "(0 stream, 1 tile, 2 LDS-ring stream, 3 GEMV, 4 persistent token-stationary "
                    "stream); the current pick is always kept")
    ap.add_argument("--max-split", type=int, default=256)
    ap.add_argument("--max-token-tiles", type=int, default=4)
    ap.add_argument("--moe", default=None,
                    help="comma list of formats: sweep the grouped call on the mixture-of-experts "
                         "layers at the --moe-batches token counts")
    ap.add_argument("--moe-batches", default="1,4,16,32,64,128,512,2048")
    ap.add_argument("--run-point", default=None,
                    help="fmt,M,N,K: only run the library's selected config of this point --reps "
                         "times over cold weight copies (a single-kernel program to profile)")
    ap.add_argument("--reps", type=int, default=8)
    ap.add_argument("--min-gain", type=float, default=0.02,
                    help="keep the current pick unless the best candidate is faster by this fraction "
                         "(timings of one run differ by about that much between candidates of equal speed)")
    args = ap.parse_args()
    sel = {"max_split": args.max_split, "max_token_tiles": args.max_token_tiles,
           "kernels": None if args.kernels is None else {int(k) for k in args.kernels.split(",")}}
    sys.path.insert(0, ROOT)
    import synth

    if args.run_point:
        f, M, N, K = args.run_point.split(",")
        M, N, K = int(M), int(N), int(K)
        pt = Point(f, M, N, K)
        c = q.select_config(f, M, N, K)
        for i in range(args.reps):
            pt.call(c, i)
        torch.cuda.synchronize()
        print(f"[tune] ran {f} M={M} N={N} K={K} x{args.reps}: {table_line(f, M, N, K, c)}", flush=True)
        return
    points = []
    for w in args.workload:
        points += synth.workload(w)
    for p in args.point:
        f, M, N, K = p.split(",")
        points.append((f, int(M), int(N), int(K)))
    points = [pt for pt in points if args.min_m <= pt[1] <= args.max_m]
    done = {}
    if args.jsonl and os.path.exists(args.jsonl):
        for ln in open(args.jsonl):
            try:
                r = json.loads(ln)
                done[r["key"]] = r
            except ValueError:
                pass
    log = open(args.jsonl, "a") if args.jsonl else None
    best = {}
    gbest = {}
    t0 = time.time()
    for fmt in (args.moe.split(",") if args.moe else []):
        for _, K, N in synth.MOE_LAYERS:
            for batch in (int(b) for b in args.moe_batches.split(",")):
                res, M = tune_grouped(fmt, N, K, batch, log=log, done=done, verbose=args.verbose)
                us, c, _ = res[0]
                cur = q.select_grouped_config(fmt, M, N, K)
                cus = next((r[0] for r in res if r[1] == cur), float("nan"))
                if cus == cus and us > cus * (1.0 - args.min_gain):
                    us, c = cus, cur
                if (fmt, M, N, K) in gbest and gbest[(fmt, M, N, K)][0] <= us:
                    continue
                gbest[(fmt, M, N, K)] = (us, c)
                print(f"[tune] grouped {fmt:9s} batch={batch:5d} max_rows={M:4d} N={N:6d} K={K:6d}: "
                      f"best {us:8.2f} us current {cus:8.2f} us | {len(res)} cands | "
                      f"{table_line(fmt, M, N, K, c, grouped=True)} [{time.time() - t0:.0f}s]", flush=True)
    for (fmt, M, N, K) in points:
        res = tune_point(fmt, M, N, K, log=log, done=done, max_cands=args.max_cands,
                         verbose=args.verbose, **sel)
        us, c, _ = res[0]
        dflt = q.select_config(fmt, M, N, K)
        dus = next((r[0] for r in res if r[1] == dflt), float("nan"))
        if dus == dus and us > dus * (1.0 - args.min_gain):
            us, c = dus, dflt
        best[(fmt, M, N, K)] = c
        print(f"[tune] {fmt:9s} M={M:5d} N={N:6d} K={K:6d}: best {us:8.2f} us "
              f"({alg_bytes(fmt, M, N, K) / us / 1e6:.3f} TB/s, {2 * M * N * K / us / 1e6:.1f} TFLOP/s) "
              f"default {dus:8.2f} us | {len(res)} cands | {table_line(fmt, M, N, K, c)} "
              f"[{time.time() - t0:.0f}s]", flush=True)
    if args.table:
        lines = {}
        if os.path.exists(args.table):
            for ln in open(args.table):
                s = ln.split("#")[0].split()
                g = bool(s) and s[0] == "grouped"
                s = s[1:] if g else s
                if len(s) == 14:
                    lines[(g, s[0], int(s[3]), int(s[1]), int(s[2]))] = ln.strip()
        for (fmt, M, N, K), c in best.items():
            lines[(False, fmt, M, N, K)] = table_line(fmt, M, N, K, c)
        for (fmt, M, N, K), (_, c) in gbest.items():
            lines[(True, fmt, M, N, K)] = table_line(fmt, M, N, K, c, grouped=True)
        hdr = [ln.rstrip("\n") for ln in open(args.table) if ln.startswith("#")] \
            if os.path.exists(args.table) else []
        with open(args.table, "w") as f:
            f.write("\n".join(hdr) + "\n")
            for k in sorted(lines):
                f.write(lines[k] + "\n")


if __name__ == "__main__":
    main()
