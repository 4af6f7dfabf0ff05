"""Build libqlinear.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m int8_gemm_linear_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqlinear.so")
DISPATCH_BENCH = os.path.join(PKG, "qlin_dispatch_bench")
TABLE = os.path.join(PKG, "configs", "qlin_mi355x.cfg")

SOURCES = [
    "qlin_api.cpp",
    "qlin_noalloc.hip",
    "qlin_reduce.hip",
    "qlin_quant.hip",
    "qlin_fused.hip",
    "qlin_stream_fp8.hip",
    "qlin_stream_int8.hip",
    "qlin_stream_block.hip",
    "qlin_tile_fp8.hip",
    "qlin_tile_h_fp8.hip",
    "qlin_tile_h_int8.hip",
    "qlin_tile_int8.hip",
    "qlin_tile_block.hip",
    "qlin_stream_lds_fp8.hip",
    "qlin_stream_lds_int8.hip",
    "qlin_stream_lds_block.hip",
    "qlin_gemv.hip",
    "qlin_stream_tok_fp8.hip",
    "qlin_stream_tok_int8.hip",
    "qlin_stream_own.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqlinear.so)")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 math stays off in all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC, "-I", BUILD]


def write_table_inc() -> str:
    """Embed the tuned config table (text) as the compiled-in default."""
    with open(TABLE) as f:
        text = f.read()
    if ")QLINTABLE" in text:
        raise ValueError("config table contains the raw-string delimiter")
    out = os.path.join(BUILD, "qlin_config_table.inc")
    body = ("// Generated from configs/qlin_mi355x.cfg by build.py.\n"
            f'static const char kDefaultTable[] = R"QLINTABLE({text})QLINTABLE";\n')
    old = open(out).read() if os.path.exists(out) else None
    if old != body:
        with open(out, "w") as f:
            f.write(body)
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libqlinear.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    write_table_inc()
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # host-side dispatch measurement program, linked against the library
    tmp = DISPATCH_BENCH + ".tmp"
    cmd = [hipcc()] + flags() + [os.path.join(PKG, "dispatch_bench.hip"), "-o", tmp, "-L", PKG,
                                 "-lqlinear", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"dispatch bench build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DISPATCH_BENCH)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
